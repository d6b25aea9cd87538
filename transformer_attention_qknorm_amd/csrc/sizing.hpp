// Workspace sizing shared by the host API and the launchers (host-only, no HIP
// types): the layout of the backward's per-row arrays and of the decode's
// split-KV partials.  Kept in one header so that the validation layer can be
// built and checked without the kernels.
#pragma once

#include <stddef.h>

namespace ncattn {

// Backward workspace: -D_i [B][H][T] fp32, padded to 256 bytes; bf16 adds
// LSE_i log2(e) of the same size right after it.
inline size_t bwd_row_bytes(int B, int T, int H) { return ((size_t)B * H * T * sizeof(float) + 255) & ~(size_t)255; }

inline size_t bwd_workspace_bytes(int B, int T, int H, int W, bool bf16) {
  (void)W;
  const size_t rows = bwd_row_bytes(B, T, H);
  return bf16 ? 2 * rows : rows;
}

// Decode: the visible keys of a sequence are cut into chunks of kDecodeChunk;
// one partial (unnormalised o [D] fp32, row max, row sum) per (b, head, chunk).
constexpr int kDecodeChunk = 128;

inline int decode_chunks_max(int T_max, int window) {
  const int span = (window < 0 || window + 1 > T_max) ? T_max : window + 1;
  return (span + kDecodeChunk - 1) / kDecodeChunk;
}

inline size_t decode_workspace_bytes(int B, int T_max, int H, int KV, int D, int window) {
  (void)KV;
  const size_t parts = (size_t)B * H * decode_chunks_max(T_max, window);
  return parts * (D + 2) * sizeof(float) + 256;
}

}  // namespace ncattn
