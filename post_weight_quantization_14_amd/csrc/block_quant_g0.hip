// Column quantizer instantiated for group width = whole row.
#define GPTQ_BQ_GW 0
#include "block_quant.inl"
