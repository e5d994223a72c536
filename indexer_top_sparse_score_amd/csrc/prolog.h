// Launch interface of the indexer prolog (prolog.hip), shared with the
// C-ABI front end.  Nothing here is exported.
#pragma once

#include "dsa_common.h"

namespace dsa {

// The indexer prolog (prolog.hip): rows of x [num_rows][D_x] through W_q
// [H_I * D_I][D_x] into MXFP8 qI / qI_scale and through W_g [H_I][D_x] into
// w, and each row's new key k_new [num_rows][D_I] normalised with gamma
// [D_I], quantised and written at its row's slot of the MXFP8 key cache kI.
struct PrologLaunch {
  RowMap rows;
  const uint16_t* x;
  const uint16_t* w_q;
  const uint16_t* w_g;
  const uint16_t* k_new;
  const uint16_t* k_gamma;
  uint8_t* qI;
  uint8_t* qI_scale;
  float* w;
  uint8_t* kI;
  int64_t kI_block_stride, kI_row_stride, kI_num_blocks;
  uint32_t* err;
  int32_t num_rows, D_x, H_I, D_I;
  float eps;
};
hipError_t launch_indexer_prolog(const PrologLaunch& a, hipStream_t s);

}  // namespace dsa
