// C ABI of libcutbce.so (declared in include/cutbce.h): argument checks, workspace layout, and the sequence of
// launches for the forward and backward of the fused full-vocabulary BCE.
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/cutbce.h"
#include "common.h"

using namespace cutbce;

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool supported(int dtype, int D) {
  if (dtype == CUTBCE_BF16) return D == 64 || D == 128 || D == 256 || D == 512;
  if (dtype == CUTBCE_F32) return D == 64 || D == 128 || D == 256;
  return false;
}

cutbce_status check_problem(const cutbce_problem* p) {
  if (!p) return CUTBCE_ERR_NULL;
  if (p->dtype != CUTBCE_F32 && p->dtype != CUTBCE_BF16) return CUTBCE_ERR_DTYPE;
  if (p->rows < 1 || p->vocab < 1 || p->nnz < 0 || p->dim < 1) return CUTBCE_ERR_SHAPE;
  if (p->rows > (int64_t)0x7fffffff - 1024 || p->vocab > (int64_t)0x7fffffff - 1024 || p->nnz > 0x7fffffffLL)
    return CUTBCE_ERR_SHAPE;
  if (!supported(p->dtype, p->dim)) return CUTBCE_ERR_UNSUPPORTED;
  return CUTBCE_OK;
}

Layout make_layout(const cutbce_problem* p) {
  Layout L;
  memset(&L, 0, sizeof L);
  L.R = p->rows;
  L.V = p->vocab;
  L.nnz = p->nnz;
  L.D = p->dim;
  L.dtype = p->dtype;
  L.esz = p->dtype == CUTBCE_BF16 ? 2 : 4;
  L.R_pad = round_up(L.R, kPad);
  L.V_pad = round_up(L.V, kPad);
  L.rows_per_wg = sweep_waves(L.dtype, L.D) * 32;
  L.items_per_wg = items_tile(L.dtype, L.D);
  L.n_rt = L.R_pad / L.rows_per_wg;
  L.n_vt = L.V_pad / L.items_per_wg;
  L.n_rs = L.R_pad / 32;
  L.n_vs = L.V_pad / 32;
  L.n_eblk = (L.V_pad + kEBlkItems - 1) / kEBlkItems;
  L.nb_r = L.n_rt * L.n_vs;
  L.nb_i = L.n_vt * L.n_rs;
  // Forward-sweep partials are indexed by unit (row tile x vocabulary split). The device picks at most
  // min(64, steps / 8) splits and at most 1024 units (choose_splits), for at most n_rt row tiles; the dE sweep's
  // halved tail tiles reuse the area (two partial sums each, fewer than min(1024, n_vt) tiles).
  const int64_t per_tile = L.n_vs / 8 < 1 ? 1 : (L.n_vs / 8 < kMaxSplits ? L.n_vs / 8 : kMaxSplits);
  int64_t units = L.n_rt * per_tile < 1024 ? L.n_rt * per_tile : 1024;
  if (units < L.n_rt) units = L.n_rt;
  const int64_t tail_tiles = L.n_vt < 1024 ? L.n_vt : 1024;
  const int64_t part_rows = (units > tail_tiles ? units : tail_tiles) * (int64_t)L.rows_per_wg;
  L.part_rows = part_rows;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.off_ctl = take(256);
  L.off_row_of = take(sizeof(int32_t) * L.R_pad);
  L.off_compact_of = take(sizeof(int32_t) * L.R);
  L.off_rptr = take(sizeof(int32_t) * 2 * L.R_pad);
  L.off_wc = take(sizeof(float) * L.R_pad);
  L.off_Hc = take((size_t)L.R_pad * L.D * L.esz);
  L.off_Hrp = take((size_t)L.R_pad * L.D * L.esz);
  L.off_sumH = take(sizeof(double) * L.D);
  L.off_sumH_part = take(sizeof(double) * L.D * (L.R_pad / 32));
  L.off_sumE = take(sizeof(double) * L.D);
  L.off_sumE_part = take(sizeof(double) * L.D * L.n_eblk);
  L.off_sum2 = take(sizeof(double) * L.D * kSumMaxGroups);
  L.off_Evp = take((size_t)L.V_pad * L.D * L.esz);
  L.off_dhpart = take(sizeof(float) * (size_t)part_rows * L.D);
  L.off_rowpart = take(sizeof(float) * 2 * (size_t)part_rows);
  L.off_metpart = take(sizeof(int32_t) * 4 * (size_t)part_rows);
  L.off_rowloss = take(sizeof(double) * L.R_pad);
  L.off_dhtmp = take(sizeof(float) * (size_t)L.R * L.D);
  L.off_estat = take(sizeof(float) * 2 * (size_t)L.n_eblk);  // E statistics: two maxima per preparation block
  L.off_rowform = take((size_t)L.R_pad);
  L.off_bptr_r = take(sizeof(int32_t) * (L.nb_r + 1));
  L.off_bfill_r = take(sizeof(int32_t) * L.nb_r);
  L.off_pairs_r = take(sizeof(int32_t) * 2 * (L.nnz > 0 ? L.nnz : 1));
  L.off_bptr_i = take(sizeof(int32_t) * (L.nb_i + 1));
  L.off_bfill_i = take(sizeof(int32_t) * L.nb_i);
  L.off_pairs_i = take(sizeof(int32_t) * 2 * (L.nnz > 0 ? L.nnz : 1));
  const int64_t nbmax = L.nb_r > L.nb_i ? L.nb_r : L.nb_i;
  L.scan_elems = (size_t)((nbmax + 1 + kScanBlock - 1) / kScanBlock + 1);
  L.off_scan = take(sizeof(int32_t) * L.scan_elems);
  L.off_cpart = take((sizeof(double) + sizeof(int32_t)) * (size_t)((L.R + 4095) / 4096));  // compaction chunks
  L.total = o;
  return L;
}

bool misaligned(const void* ptr, size_t a) { return ptr && ((uintptr_t)ptr % a) != 0; }

cutbce_status hip_status(hipError_t e) { return e == hipSuccess ? CUTBCE_OK : CUTBCE_ERR_HIP; }

// Opt-in sweep timing (see cutbce_profile_enable).
struct ProfRec {
  hipEvent_t a, b;
  int kind;
};
bool g_prof_on = false;
std::vector<ProfRec> g_prof_pool;
size_t g_prof_used = 0;
constexpr size_t kProfMax = 65536;

ProfRec* prof_begin(int kind, hipStream_t st) {
  if (!g_prof_on || g_prof_used >= kProfMax) return nullptr;
  if (g_prof_used == g_prof_pool.size()) {
    ProfRec r;
    if (hipEventCreate(&r.a) != hipSuccess) return nullptr;
    if (hipEventCreate(&r.b) != hipSuccess) {
      (void)hipEventDestroy(r.a);
      return nullptr;
    }
    g_prof_pool.push_back(r);
  }
  ProfRec* r = &g_prof_pool[g_prof_used];
  if (hipEventRecord(r->a, st) != hipSuccess) return nullptr;
  r->kind = kind;
  ++g_prof_used;
  return r;
}

void prof_end(ProfRec* r, hipStream_t st) {
  if (r && hipEventRecord(r->b, st) != hipSuccess) r->kind = -1;
}

hipError_t timed_rows(const Layout& L, char* ws, const void* E, bool with_dh, bool met, hipStream_t st) {
  ProfRec* r = prof_begin(0, st);
  hipError_t e = launch_rows_sweep(L, ws, E, with_dh, met, !kGatherPositives, st);
  prof_end(r, st);
  return e;
}

hipError_t timed_items(const Layout& L, char* ws, const void* E, const float* g, void* dE, hipStream_t st) {
  ProfRec* r = prof_begin(1, st);
  hipError_t e = launch_items_sweep(L, ws, E, g, dE, st);
  prof_end(r, st);
  return e;
}

#define TRY(x)                                 \
  do {                                         \
    hipError_t e_ = (x);                       \
    if (e_ != hipSuccess) return CUTBCE_ERR_HIP; \
  } while (0)

cutbce_status check_common(const cutbce_problem* p, const void* H, const void* E, const int32_t* ro,
                           const int32_t* ids, const uint8_t* mask, void* ws, size_t ws_bytes, Layout* L) {
  cutbce_status s = check_problem(p);
  if (s != CUTBCE_OK) return s;
  if (!H || !E || !ro || !mask || !ws || (p->nnz > 0 && !ids)) return CUTBCE_ERR_NULL;
  if (misaligned(H, 16) || misaligned(E, 16) || misaligned(ws, 256) || misaligned(ro, 4) || misaligned(ids, 4))
    return CUTBCE_ERR_ALIGN;
  *L = make_layout(p);
  if (ws_bytes < L->total) return CUTBCE_ERR_WORKSPACE;
  return CUTBCE_OK;
}

// Scratch of cutbce_forward_noalloc: a device array of the library (one per GPU, held until the process ends).
// In host code `scratch` names a host-side stand-in, never the device memory: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed to kernels.
static __device__ __align__(256) char scratch[CUTBCE_NOALLOC_SCRATCH_BYTES];
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];

// Device address of the current device's scratch array (looked up on the first call on that device).
cutbce_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CUTBCE_ERR_HIP;
  if (dev < 0 || dev >= kScratchDevices) return CUTBCE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return CUTBCE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CUTBCE_OK;
}

}  // namespace

extern "C" {

int cutbce_version(void) { return 200; }

const char* cutbce_status_string(cutbce_status s) {
  switch (s) {
    case CUTBCE_OK: return "ok";
    case CUTBCE_ERR_NULL: return "a required pointer is NULL";
    case CUTBCE_ERR_SHAPE: return "invalid sizes";
    case CUTBCE_ERR_DTYPE: return "unknown element type";
    case CUTBCE_ERR_ALIGN: return "misaligned pointer";
    case CUTBCE_ERR_WORKSPACE: return "workspace too small";
    case CUTBCE_ERR_UNSUPPORTED: return "unsupported (dtype, dim)";
    case CUTBCE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

cutbce_status cutbce_workspace_size(const cutbce_problem* p, size_t* bytes) {
  cutbce_status s = check_problem(p);
  if (s != CUTBCE_OK) return s;
  if (!bytes) return CUTBCE_ERR_NULL;
  *bytes = make_layout(p).total;
  return CUTBCE_OK;
}

cutbce_status cutbce_forward(const cutbce_problem* p, const void* H, const void* E, const int32_t* row_offsets,
                             const int32_t* item_ids, const uint8_t* row_mask, const float* row_weight,
                             float* loss, float* row_loss, float* dh_saved, int32_t* metrics, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Layout L;
  cutbce_status s = check_common(p, H, E, row_offsets, item_ids, row_mask, workspace, workspace_bytes, &L);
  if (s != CUTBCE_OK) return s;
  if (!loss) return CUTBCE_ERR_NULL;
  if (misaligned(dh_saved, 16) || misaligned(loss, 4) || misaligned(row_loss, 4) || misaligned(metrics, 4) ||
      misaligned(row_weight, 4))
    return CUTBCE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const bool with_dh = dh_saved != nullptr;
  TRY(launch_compact(L, ws, row_mask, row_weight, row_offsets, st));
  TRY(launch_prep_h(L, ws, H, false, st));
  TRY(launch_prep_e(L, ws, E, with_dh, st));
  // positives gathered by the finish; the sweep's buckets are empty, or, with Cut Metrics, only counted
  TRY(kGatherPositives && !metrics ? launch_no_row_buckets(L, ws, st) : launch_buckets(L, ws, item_ids, true, st));
  TRY(timed_rows(L, ws, E, with_dh, metrics != nullptr, st));
  TRY(launch_rows_finish(L, ws, H, row_mask, loss, row_loss, dh_saved, with_dh, metrics,
                         kGatherPositives ? E : nullptr, item_ids, st));
  return CUTBCE_OK;
}

cutbce_status cutbce_forward_noalloc(const cutbce_problem* p, const void* H, const void* E,
                                     const int32_t* row_offsets, const int32_t* item_ids, const uint8_t* row_mask,
                                     const float* row_weight, float* loss, float* row_loss, float* dh_saved,
                                     int32_t* metrics, void* stream) {
  cutbce_status s = check_problem(p);
  if (s != CUTBCE_OK) return s;
  if (make_layout(p).total > (size_t)CUTBCE_NOALLOC_SCRATCH_BYTES) return CUTBCE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((s = scratch_of_current_device(&ws)) != CUTBCE_OK) return s;
  // every kernel of the forward initialises what it reads from the workspace, so the previous call's contents
  // do not matter
  return cutbce_forward(p, H, E, row_offsets, item_ids, row_mask, row_weight, loss, row_loss, dh_saved, metrics, ws,
                        (size_t)CUTBCE_NOALLOC_SCRATCH_BYTES, stream);
}

// reuse: the workspace holds the row compaction and H preparation of a cutbce_forward on the same inputs
static cutbce_status backward_impl(const cutbce_problem* p, const void* H, const void* E, const int32_t* row_offsets,
                                   const int32_t* item_ids, const uint8_t* row_mask, const float* row_weight,
                                   const float* grad_loss, const float* dh_saved, void* dH, void* dE, void* workspace,
                                   size_t workspace_bytes, void* stream, bool reuse) {
  Layout L;
  cutbce_status s = check_common(p, H, E, row_offsets, item_ids, row_mask, workspace, workspace_bytes, &L);
  if (s != CUTBCE_OK) return s;
  if (!grad_loss) return CUTBCE_ERR_NULL;
  if (misaligned(dh_saved, 16) || misaligned(dH, 16) || misaligned(dE, 16) || misaligned(grad_loss, 4) ||
      misaligned(row_weight, 4))
    return CUTBCE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (!dH && !dE) return CUTBCE_OK;
  if (!reuse) {
    TRY(launch_compact(L, ws, row_mask, row_weight, row_offsets, st));
    TRY(launch_prep_h(L, ws, H, dE != nullptr, st));
  } else if (dE) {
    TRY(launch_prep_hrp(L, ws, H, st));
  }
  if (dE) {
    TRY(launch_buckets(L, ws, item_ids, false, st));
    TRY(timed_items(L, ws, E, grad_loss, dE, st));
  }
  if (dH) {
    if (dh_saved) {
      TRY(launch_scale_dh(L, dh_saved, grad_loss, dH, st));
    } else {
      float* tmp = (float*)(ws + L.off_dhtmp);
      TRY(launch_prep_e(L, ws, E, true, st));
      TRY(kGatherPositives ? launch_no_row_buckets(L, ws, st) : launch_buckets(L, ws, item_ids, true, st));
      TRY(timed_rows(L, ws, E, true, false, st));
      TRY(launch_rows_finish(L, ws, H, row_mask, nullptr, nullptr, tmp, true, nullptr,
                             kGatherPositives ? E : nullptr, item_ids, st));
      TRY(launch_scale_dh(L, tmp, grad_loss, dH, st));
    }
  }
  return CUTBCE_OK;
}

cutbce_status cutbce_backward(const cutbce_problem* p, const void* H, const void* E, const int32_t* row_offsets,
                              const int32_t* item_ids, const uint8_t* row_mask, const float* row_weight,
                              const float* grad_loss, const float* dh_saved, void* dH, void* dE, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return backward_impl(p, H, E, row_offsets, item_ids, row_mask, row_weight, grad_loss, dh_saved, dH, dE, workspace,
                       workspace_bytes, stream, false);
}

cutbce_status cutbce_backward_reuse(const cutbce_problem* p, const void* H, const void* E,
                                    const int32_t* row_offsets, const int32_t* item_ids, const uint8_t* row_mask,
                                    const float* row_weight, const float* grad_loss, const float* dh_saved, void* dH,
                                    void* dE, void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(p, H, E, row_offsets, item_ids, row_mask, row_weight, grad_loss, dh_saved, dH, dE, workspace,
                       workspace_bytes, stream, true);
}

cutbce_status cutbce_validate_targets(const cutbce_problem* p, const int32_t* row_offsets, const int32_t* item_ids,
                                      int32_t* bad, void* stream) {
  cutbce_status s = check_problem(p);
  if (s != CUTBCE_OK) return s;
  if (!row_offsets || !bad || (p->nnz > 0 && !item_ids)) return CUTBCE_ERR_NULL;
  if (misaligned(row_offsets, 4) || misaligned(item_ids, 4) || misaligned(bad, 4)) return CUTBCE_ERR_ALIGN;
  return hip_status(launch_validate(p->rows, p->vocab, p->nnz, row_offsets, item_ids, bad, (hipStream_t)stream));
}

cutbce_status cutbce_topk(const cutbce_problem* p, const void* H, const void* E, const int32_t* row_offsets,
                          const int32_t* item_ids, const uint8_t* row_mask, int32_t k, float* top_vals,
                          int32_t* top_ids, int32_t* hits, void* workspace, size_t workspace_bytes, void* stream) {
  Layout L;
  cutbce_status s = check_common(p, H, E, row_offsets, item_ids, row_mask, workspace, workspace_bytes, &L);
  if (s != CUTBCE_OK) return s;
  if (!top_vals || !top_ids) return CUTBCE_ERR_NULL;
  if (k < 1 || k > kTopKMax || k > p->vocab) return CUTBCE_ERR_SHAPE;
  if (misaligned(top_vals, 4) || misaligned(top_ids, 4) || misaligned(hits, 4)) return CUTBCE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int kt = kTopKMax;
  TRY(launch_compact(L, ws, row_mask, nullptr, row_offsets, st));
  TRY(launch_prep_h(L, ws, H, false, st));
  TRY(launch_fill_i32((int32_t*)(ws + L.off_bptr_r), L.nb_r + 1, 0, st));  // no positive buckets
  {
    ProfRec* r = prof_begin(2, st);
    const hipError_t e = launch_topk_sweep(L, ws, E, kt, st);
    prof_end(r, st);
    TRY(e);
  }
  TRY(launch_topk_finish(L, ws, row_mask, item_ids, kt, k, top_vals, top_ids, hits, st));
  return CUTBCE_OK;
}

cutbce_status cutbce_targets_to_csr(int64_t rows, int32_t slots, const int32_t* targets, int32_t pad_id,
                                    int32_t* row_offsets, int32_t* item_ids, void* stream) {
  if (rows < 1 || slots < 0 || rows > (int64_t)0x7fffffff - 1024 || rows * (int64_t)slots > 0x7fffffffLL)
    return CUTBCE_ERR_SHAPE;
  if (!row_offsets || (slots > 0 && (!targets || !item_ids))) return CUTBCE_ERR_NULL;
  if (misaligned(targets, 4) || misaligned(row_offsets, 4) || misaligned(item_ids, 4)) return CUTBCE_ERR_ALIGN;
  return hip_status(launch_targets_to_csr(rows, slots, targets, pad_id, row_offsets, item_ids, (hipStream_t)stream));
}

cutbce_status cutbce_profile_enable(int on) {
  g_prof_on = on != 0;
  g_prof_used = 0;
  return CUTBCE_OK;
}

cutbce_status cutbce_profile_read(double* ms, int64_t* launches, int n_kinds) {
  if (!ms || !launches || n_kinds < 0) return CUTBCE_ERR_NULL;
  for (int k = 0; k < n_kinds; ++k) {
    ms[k] = 0.0;
    launches[k] = 0;
  }
  cutbce_status st = CUTBCE_OK;
  for (size_t i = 0; i < g_prof_used; ++i) {
    ProfRec& r = g_prof_pool[i];
    if (r.kind < 0 || r.kind >= n_kinds) continue;
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
      st = CUTBCE_ERR_HIP;
      continue;
    }
    ms[r.kind] += t;
    launches[r.kind] += 1;
  }
  g_prof_used = 0;
  return st;
}

}  // extern "C"
