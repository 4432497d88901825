// Column quantizer instantiated for group width 16.
#define GPTQ_BQ_GW 16
#include "block_quant.inl"
