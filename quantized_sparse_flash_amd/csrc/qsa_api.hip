// qsa_api.hip -- the C ABI of libqsa (declared in include/qsa.h).
//
// Every entry point validates its arguments on the host, before anything is
// enqueued, then launches the gfx950 kernels on the caller's stream.  The
// library allocates nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "qsa.h"
#include "qsa_launch.h"

// Device scratch of qsa_flash_noalloc: one copy per GPU, alive until the
// process ends.  In host code `scratch` is only a stand-in for the symbol:
// its device address comes from hipGetSymbolAddress (see scratch_ptr).
static __device__ __align__(256) uint8_t scratch[QSA_NOALLOC_SCRATCH_BYTES];


namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape checks shared by all entry points.  Returns QSA_OK or an error.
int check_shape(const qsa_shape* s) {
  if (!s) return QSA_ERR_ARG;
  if (s->heads_per_group != QSA_HEADS_PER_GROUP || s->head_dim != QSA_HEAD_DIM)
    return QSA_ERR_UNSUPPORTED;
  if (s->budget < 1 || s->budget > QSA_MAX_BUDGET) return QSA_ERR_UNSUPPORTED;
  if (s->T < 1 || s->pos0 < 0 || s->n_groups < 1) return QSA_ERR_SHAPE;
  if (s->n_cells < (int64_t)s->pos0 + s->T) return QSA_ERR_SHAPE;
  // cell indices are int32 on the device; grids are 1-D
  if (s->n_cells > INT32_MAX || (int64_t)s->pos0 + s->T > INT32_MAX) return QSA_ERR_SHAPE;
  const int64_t rows = (int64_t)s->T * s->n_groups;
  const int64_t kc = (s->budget + QSA_CHUNK - 1) / QSA_CHUNK;
  if (rows > INT32_MAX / 4 || rows * kc > INT32_MAX / 4) return QSA_ERR_SHAPE;
  if ((int64_t)s->n_groups * QSA_HEADS_PER_GROUP * s->T > INT32_MAX / 4) return QSA_ERR_SHAPE;
  return QSA_OK;
}

bool any_above_budget(const qsa_shape* s) { return (int64_t)s->pos0 + s->T > s->budget; }

// Tokens [0, t_id) of the chunk are under budget (identity selection).
int identity_tokens(const qsa_shape* s) {
  const int64_t under = (int64_t)s->budget - s->pos0;
  return (int)(under < 0 ? 0 : (under > s->T ? s->T : under));
}

int launch_status(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_LAUNCH; }

// How a fused call runs, and its workspace.  Tokens under budget share a
// prefix of cells: the tiled path dequantises it once (the chunk images,
// plus room for the split pieces of a tiled grid that leaves CUs idle) and
// attends from it.  Rows above budget run on the row kernel, one wavefront
// per row; when they are few (at most kRowPiecesMax) they run instead as
// row pieces (one wavefront per piece of a few 64-cell chunks, about
// kPieceWaves wavefronts in all) plus the merge, which fill the GPU where
// a lone row would take the row kernel ~100 us.  Their records follow the
// tiled part.  When the whole call has at most kAllPiecesMax rows and some
// above budget, every token runs that way (the few tokens under budget
// gain nothing from the tiled path's two extra launches), with the records
// alone in the workspace.  The public calls ask for the whole workspace of
// the route (qsa_flash_workspace_bytes); qsa_flash_noalloc asks only for
// the chunk images, and takes a pieces route only when its scratch holds
// that route's records.
//
// Both limits count (token, group) rows.  Measured at pos0 30000: pieces
// took 62 / 76 / 101 us for 300 / 400 / 600 rows against 104 us on the row
// kernel, and 130 against 106 us for 1000 rows (one piece per row: only
// the merge added).
constexpr int64_t kRowPiecesMax = 512;
constexpr int64_t kAllPiecesMax = 256;

enum class Route { kRows, kRowPieces, kAllPieces };

Route route_of(const qsa_shape* s) {
  const int64_t t_above = s->T - identity_tokens(s);
  if (t_above <= 0) return Route::kRows;  // no row above budget
  if ((int64_t)s->T * s->n_groups <= kAllPiecesMax) return Route::kAllPieces;
  if (t_above * s->n_groups <= kRowPiecesMax) return Route::kRowPieces;
  return Route::kRows;
}
// Chunks per record of the row pieces of `rows` (token, group) rows: about
// kPieceWaves wavefronts in all, one per SIMD, a piece at least one chunk
// (measured against 512 to 4096: fewer, longer pieces amortise the staged
// pipeline's start; fewer wavefronts than SIMDs leave the GPU idle).
constexpr int64_t kPieceWaves = 1024;
int pieces_cpr(int64_t rows, int kc) {
  const int64_t c = (rows * kc + kPieceWaves - 1) / kPieceWaves;
  return (int)(c < 1 ? 1 : (c > kc ? kc : c));
}
int64_t record_bytes(const qsa_shape* s, int64_t tokens) {
  const int kc = (s->budget + QSA_CHUNK - 1) / QSA_CHUNK;
  const int cpr = pieces_cpr(tokens * s->n_groups, kc);
  const int64_t kcr = (kc + cpr - 1) / cpr;
  return tokens * kcr * s->n_groups * QSA_HEADS_PER_GROUP * QSA_PART_STRIDE * 4;
}
int64_t tile_part_bytes(const qsa_shape* s) {
  const int64_t b = qsa::tile_workspace_bytes(s->n_groups, identity_tokens(s), s->pos0);
  return (b + 255) / 256 * 256;
}
int64_t full_workspace(const qsa_shape* s) {
  switch (route_of(s)) {
    case Route::kAllPieces: return record_bytes(s, s->T);
    case Route::kRowPieces: return tile_part_bytes(s) + record_bytes(s, s->T - identity_tokens(s));
    default: return qsa::tile_workspace_bytes(s->n_groups, identity_tokens(s), s->pos0);
  }
}
// The route a call with workspace_bytes of scratch takes: a pieces route
// only when the scratch holds its workspace.
Route route_with(const qsa_shape* s, int64_t workspace_bytes) {
  const Route r = route_of(s);
  if (r != Route::kRows && workspace_bytes < full_workspace(s)) return Route::kRows;
  return r;
}
int64_t min_workspace(const qsa_shape* s) {
  return qsa::tile_workspace_min_bytes(s->n_groups, identity_tokens(s), s->pos0);
}

}  // namespace

extern "C" {

const char* qsa_status_string(int status) {
  switch (status) {
    case QSA_OK: return "ok";
    case QSA_ERR_ARG: return "invalid argument (NULL or misaligned pointer)";
    case QSA_ERR_UNSUPPORTED: return "unsupported configuration (heads_per_group, head_dim or budget)";
    case QSA_ERR_SHAPE: return "invalid shape (T, pos0, n_groups or n_cells)";
    case QSA_ERR_LAUNCH: return "kernel launch failed";
    case QSA_ERR_TOO_LARGE:
      return "shape needs more scratch than qsa_flash_noalloc holds (QSA_NOALLOC_SCRATCH_BYTES)";
    case QSA_ERR_DEVICE: return "HIP device query failed";
    default: return "unknown status";
  }
}

int64_t qsa_part_elems(const qsa_shape* s) {
  if (check_shape(s) != QSA_OK) return 0;
  const int64_t kc = (s->budget + QSA_CHUNK - 1) / QSA_CHUNK;
  return (int64_t)s->T * kc * s->n_groups * QSA_HEADS_PER_GROUP * QSA_PART_STRIDE;
}

int qsa_score(const qsa_shape* s, int32_t index_dim, const float* qidx, const float* pooled,
              float* scores, void* stream) {
  int rc = check_shape(s);
  if (rc != QSA_OK) return rc;
  if (index_dim < 4 || index_dim > QSA_MAX_INDEX_DIM || index_dim % 4 != 0)
    return QSA_ERR_UNSUPPORTED;
  if (!any_above_budget(s)) return QSA_OK;  // no row reads scores
  if (!qidx || !pooled || !scores) return QSA_ERR_ARG;
  if (!aligned(qidx, 16) || !aligned(pooled, 16) || !aligned(scores, 16)) return QSA_ERR_ARG;
  return launch_status(qsa::launch_score(qidx, pooled, scores, s->T, s->pos0, s->n_groups,
                                         s->budget, s->n_cells, index_dim,
                                         (hipStream_t)stream));
}

int qsa_topk(const qsa_shape* s, const float* scores, int32_t* ids, void* stream) {
  int rc = check_shape(s);
  if (rc != QSA_OK) return rc;
  if (!ids || !aligned(ids, 4)) return QSA_ERR_ARG;
  if (any_above_budget(s) && (!scores || !aligned(scores, 4))) return QSA_ERR_ARG;
  return launch_status(qsa::launch_topk(scores, ids, s->T, s->pos0, s->n_groups, s->budget,
                                        s->n_cells, (hipStream_t)stream));
}

int64_t qsa_flash_workspace_bytes(const qsa_shape* s) {
  if (check_shape(s) != QSA_OK) return 0;
  return full_workspace(s);
}

}  // extern "C"

namespace {

// Host-side checks and argument packing shared by the qsa_flash entry points.
int flash_args(const qsa_shape* s, const qsa_f16* q, const int8_t* kq, const qsa_f16* ksc,
               const int8_t* vq, const qsa_f16* vsc, const int32_t* ids, qsa_f16* out,
               float* part, qsa::RowArgs* a) {
  int rc = check_shape(s);
  if (rc != QSA_OK) return rc;
  if (!kq || !ksc || !vq || !vsc) return QSA_ERR_ARG;
  if (!aligned(kq, 16) || !aligned(vq, 16) || !aligned(ksc, 8) || !aligned(vsc, 8))
    return QSA_ERR_ARG;
  a->q = reinterpret_cast<const _Float16*>(q);
  a->kq = kq;
  a->ksc = reinterpret_cast<const _Float16*>(ksc);
  a->vq = vq;
  a->vsc = reinterpret_cast<const _Float16*>(vsc);
  a->ids = ids;
  a->out = reinterpret_cast<_Float16*>(out);
  a->part = part;
  a->T = s->T;
  a->pos0 = s->pos0;
  a->G = s->n_groups;
  a->budget = s->budget;
  a->KC = (s->budget + QSA_CHUNK - 1) / QSA_CHUNK;
  a->cpr = 1;
  a->n_items = 0;
  a->n_cells = s->n_cells;
  return QSA_OK;
}

int check_workspace(const void* workspace, int64_t workspace_bytes, int64_t need) {
  if (need > 0 && (!workspace || !aligned(workspace, 256) || workspace_bytes < need))
    return QSA_ERR_ARG;
  return QSA_OK;
}

// q, ids and out of a fused call (attention half).
int check_attend(const qsa_shape* s, const qsa_f16* q, const int32_t* ids, const qsa_f16* out) {
  if (!q || !aligned(q, 16)) return QSA_ERR_ARG;
  if (any_above_budget(s) && (!ids || !aligned(ids, 4))) return QSA_ERR_ARG;
  if (!out || !aligned(out, 16)) return QSA_ERR_ARG;
  return QSA_OK;
}

int prepare_impl(const qsa_shape* s, const int8_t* kq, const qsa_f16* ksc, const int8_t* vq,
                 const qsa_f16* vsc, void* workspace, int64_t workspace_bytes, void* stream,
                 int64_t need) {
  qsa::RowArgs a;
  int rc = flash_args(s, nullptr, kq, ksc, vq, vsc, nullptr, nullptr, nullptr, &a);
  if (rc == QSA_OK) rc = check_workspace(workspace, workspace_bytes, need);
  if (rc != QSA_OK) return rc;
  if (route_with(s, workspace_bytes) == Route::kAllPieces) return QSA_OK;  // nothing to prepare
  return launch_status(qsa::launch_tile_prepare(a, identity_tokens(s), workspace,
                                                workspace_bytes, (hipStream_t)stream));
}

int attend_impl(const qsa_shape* s, const qsa_f16* q, const int8_t* kq, const qsa_f16* ksc,
                const int8_t* vq, const qsa_f16* vsc, const int32_t* ids, qsa_f16* out,
                void* workspace, int64_t workspace_bytes, void* stream, int64_t need) {
  qsa::RowArgs a;
  int rc = flash_args(s, q, kq, ksc, vq, vsc, ids, out, nullptr, &a);
  if (rc == QSA_OK) rc = check_attend(s, q, ids, out);
  if (rc == QSA_OK) rc = check_workspace(workspace, workspace_bytes, need);
  if (rc != QSA_OK) return rc;
  // tokens under budget (a prefix of the chunk) see a common prefix of
  // cells, dequantised once into the workspace and shared by the tiled
  // kernel; tokens above budget gather their own ids row by row
  const int t_id = identity_tokens(s);
  const int64_t H = (int64_t)s->n_groups * QSA_HEADS_PER_GROUP;
  hipStream_t st = (hipStream_t)stream;
  // tokens [t0, T) as a shape of their own: row-piece records in the
  // workspace from byte `off`, then the merge into out
  auto piece_tokens = [&](int t0, int64_t off) {
    qsa::RowArgs b = a;
    b.q = a.q + (int64_t)t0 * H * QSA_HEAD_DIM;
    b.out = a.out + (int64_t)t0 * H * QSA_HEAD_DIM;
    if (a.ids) b.ids = a.ids + (int64_t)t0 * s->n_groups * s->budget;
    b.T = s->T - t0;
    b.pos0 = s->pos0 + t0;
    b.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + off);
    b.cpr = pieces_cpr((int64_t)b.T * s->n_groups, b.KC);
    // one chunk per record: the split kernel, which loads its chunk at once
    // (the same record layout); longer pieces: the staged row kernel
    int r = launch_status(b.cpr == 1 ? qsa::launch_flash_rows(b, true, 0, st)
                                     : qsa::launch_flash_row_pieces(b, st));
    if (r != QSA_OK) return r;
    return launch_status(
        qsa::launch_merge(b.part, b.out, b.T, (int)H, b.pos0, s->budget, b.cpr, st));
  };
  const Route route = route_with(s, workspace_bytes);
  if (route == Route::kAllPieces) return piece_tokens(0, 0);
  rc = launch_status(qsa::launch_tile_attend(a, t_id, workspace, workspace_bytes, st));
  if (rc != QSA_OK) return rc;
  if (route == Route::kRowPieces) return piece_tokens(t_id, tile_part_bytes(s));
  return launch_status(qsa::launch_flash_rows(a, false, t_id, st));
}

int flash_impl(const qsa_shape* s, const qsa_f16* q, const int8_t* kq, const qsa_f16* ksc,
               const int8_t* vq, const qsa_f16* vsc, const int32_t* ids, qsa_f16* out,
               float* part, void* workspace, int64_t workspace_bytes, void* stream,
               int64_t need) {
  qsa::RowArgs a;
  int rc = flash_args(s, q, kq, ksc, vq, vsc, ids, out, part, &a);
  if (rc != QSA_OK) return rc;
  if (part) {  // split mode: per-chunk partial records, every row by the row kernel
    if (!q || !aligned(q, 16) || !aligned(part, 16)) return QSA_ERR_ARG;
    if (any_above_budget(s) && (!ids || !aligned(ids, 4))) return QSA_ERR_ARG;
    return launch_status(qsa::launch_flash_rows(a, true, 0, (hipStream_t)stream));
  }
  rc = check_attend(s, q, ids, out);
  if (rc == QSA_OK) rc = check_workspace(workspace, workspace_bytes, need);
  if (rc != QSA_OK) return rc;
  rc = prepare_impl(s, kq, ksc, vq, vsc, workspace, workspace_bytes, stream, need);
  if (rc != QSA_OK) return rc;
  return attend_impl(s, q, kq, ksc, vq, vsc, ids, out, workspace, workspace_bytes, stream, need);
}

}  // namespace

extern "C" {

int qsa_flash_prepare(const qsa_shape* s, const int8_t* kq, const qsa_f16* ksc,
                      const int8_t* vq, const qsa_f16* vsc, void* workspace,
                      int64_t workspace_bytes, void* stream) {
  const int rc = check_shape(s);
  if (rc != QSA_OK) return rc;
  return prepare_impl(s, kq, ksc, vq, vsc, workspace, workspace_bytes, stream, full_workspace(s));
}

int qsa_flash_attend(const qsa_shape* s, const qsa_f16* q, const int8_t* kq,
                     const qsa_f16* ksc, const int8_t* vq, const qsa_f16* vsc,
                     const int32_t* ids, qsa_f16* out, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  const int rc = check_shape(s);
  if (rc != QSA_OK) return rc;
  return attend_impl(s, q, kq, ksc, vq, vsc, ids, out, workspace, workspace_bytes, stream,
                     full_workspace(s));
}

int qsa_flash(const qsa_shape* s, const qsa_f16* q, const int8_t* kq, const qsa_f16* ksc,
              const int8_t* vq, const qsa_f16* vsc, const int32_t* ids, qsa_f16* out,
              float* part, void* workspace, int64_t workspace_bytes, void* stream) {
  const int rc = check_shape(s);
  if (rc != QSA_OK) return rc;
  return flash_impl(s, q, kq, ksc, vq, vsc, ids, out, part, workspace, workspace_bytes, stream,
                    part ? 0 : full_workspace(s));
}

int qsa_merge(const qsa_shape* s, const float* part, qsa_f16* out, void* stream) {
  int rc = check_shape(s);
  if (rc != QSA_OK) return rc;
  if (!part || !out || !aligned(part, 16) || !aligned(out, 16)) return QSA_ERR_ARG;
  return launch_status(qsa::launch_merge(part, reinterpret_cast<_Float16*>(out), s->T,
                                         s->n_groups * QSA_HEADS_PER_GROUP,
                                         s->pos0, s->budget, 1, (hipStream_t)stream));
}

int qsa_quantize(int64_t n_rows, int32_t dim, const qsa_f16* x, int8_t* codes,
                 qsa_f16* scales, void* stream) {
  if (dim != QSA_HEAD_DIM) return QSA_ERR_UNSUPPORTED;
  // one workgroup per 16 rows on a 1-D grid
  if (n_rows < 0 || n_rows > (int64_t)INT32_MAX * 16) return QSA_ERR_SHAPE;
  if (n_rows == 0) return QSA_OK;
  if (!x || !codes || !scales || !aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 2))
    return QSA_ERR_ARG;
  return launch_status(qsa::launch_quantize(reinterpret_cast<const _Float16*>(x), codes,
                                            reinterpret_cast<_Float16*>(scales), n_rows,
                                            (hipStream_t)stream));
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once resolved

// Device address of the current device's copy of `scratch`, resolved on the
// first call on that device (with it current) and kept; nullptr on failure.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int qsa_flash_noalloc(const qsa_shape* s, const qsa_f16* q, const int8_t* kq,
                      const qsa_f16* ksc, const int8_t* vq, const qsa_f16* vsc,
                      const int32_t* ids, qsa_f16* out, float* part, void* stream) {
  // every host-side check of qsa_flash first (nothing touches the device)
  qsa::RowArgs a;
  int rc = flash_args(s, q, kq, ksc, vq, vsc, ids, out, part, &a);
  if (rc != QSA_OK) return rc;
  if (part) {
    if (!q || !aligned(q, 16) || !aligned(part, 16)) return QSA_ERR_ARG;
    if (any_above_budget(s) && (!ids || !aligned(ids, 4))) return QSA_ERR_ARG;
  } else {
    rc = check_attend(s, q, ids, out);
    if (rc != QSA_OK) return rc;
  }
  const int64_t need = part ? 0 : min_workspace(s);
  if (need > QSA_NOALLOC_SCRATCH_BYTES) return QSA_ERR_TOO_LARGE;
  // the scratch holds the chunk images, and the row-piece records of a route
  // that uses them when the route's whole workspace fits (with no token
  // under budget, only then is it needed)
  const int64_t full = part ? 0 : full_workspace(s);
  const bool use = need > 0 || (full > 0 && full <= QSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (use) {
    ws = scratch_ptr();
    if (!ws) return QSA_ERR_DEVICE;
  }
  return flash_impl(s, q, kq, ksc, vq, vsc, ids, out, part, ws,
                    use ? (int64_t)QSA_NOALLOC_SCRATCH_BYTES : 0, stream, need);
}

}  // extern "C"
