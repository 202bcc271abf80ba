// qsa_launch.h -- host-side launchers of the QSA kernels (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Arguments of the attention kernels (pointers are device pointers).
struct RowArgs {
  const _Float16* q;
  const int8_t* kq;
  const _Float16* ksc;
  const int8_t* vq;
  const _Float16* vsc;
  const int32_t* ids;
  _Float16* out;
  float* part;
  int T, pos0, G, budget, KC, n_items;
  int cpr;  // chunks per record of the row pieces (launch_flash_row_pieces)
  int64_t n_cells;
};

// Selection scores of the rows above budget: scores[t][g][c] for c < n_kv(t).
hipError_t launch_score(const float* qidx, const float* pooled, float* scores, int T, int pos0,
                        int G, int budget, int64_t n_cells, int dim, hipStream_t stream);
hipError_t launch_topk(const float* scores, int32_t* ids, int T, int pos0, int G, int budget,
                       int64_t n_cells, hipStream_t stream);
// Merge of records that cover cpr chunks each (1: the split-mode records).
hipError_t launch_merge(const float* part, _Float16* out, int T, int H, int pos0, int budget,
                        int cpr, hipStream_t stream);
// K/V quantiser: `rows` fp16 rows of 256 dims -> int8 codes and 4 fp16
// scales per row.
hipError_t launch_quantize(const _Float16* x, int8_t* codes, _Float16* scales, int64_t rows,
                           hipStream_t stream);
// Row kernels: one wavefront per (token, group) row for tokens [t_begin, T),
// all of which must be above budget (fused), or per (token, group, chunk)
// for all tokens (split mode).
hipError_t launch_flash_rows(const RowArgs& a, bool split, int t_begin, hipStream_t stream);
// Row pieces: one wavefront per (token, group, piece of a.cpr chunks) of
// every token, each writing that piece's (o, m, l) record into a.part
// ([T][ceil(KC / cpr)][G*12][258]); the last token must be above budget.
hipError_t launch_flash_row_pieces(const RowArgs& a, hipStream_t stream);
// Tile path: fused attention of tokens [0, t_count), all under budget.
// launch_tile_prepare dequantises cells [0, pos0 + t_count) of every group
// into `ws` (ws_bytes bytes, at least tile_workspace_min_bytes) and clears
// the split pieces' counters; launch_tile_attend then attends from it.
// Both take the same ws_bytes: it decides how many of the longest blocks
// run as two merged pieces (all that tile_workspace_bytes provides for).
int64_t tile_workspace_bytes(int G, int t_count, int pos0);
int64_t tile_workspace_min_bytes(int G, int t_count, int pos0);
hipError_t launch_tile_prepare(const RowArgs& a, int t_count, void* ws, int64_t ws_bytes,
                               hipStream_t stream);
hipError_t launch_tile_attend(const RowArgs& a, int t_count, void* ws, int64_t ws_bytes,
                              hipStream_t stream);

}  // namespace qsa
