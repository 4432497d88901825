// Column quantizer instantiated for group width 128.
#define GPTQ_BQ_GW 128
#include "block_quant.inl"
