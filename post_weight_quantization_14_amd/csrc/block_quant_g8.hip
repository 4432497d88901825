// Column quantizer instantiated for group width 8.
#define GPTQ_BQ_GW 8
#include "block_quant.inl"
