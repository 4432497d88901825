// Column quantizer instantiated for group width 32.
#define GPTQ_BQ_GW 32
#include "block_quant.inl"
