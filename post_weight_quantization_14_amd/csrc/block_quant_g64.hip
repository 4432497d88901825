// Column quantizer instantiated for group width 64.
#define GPTQ_BQ_GW 64
#include "block_quant.inl"
