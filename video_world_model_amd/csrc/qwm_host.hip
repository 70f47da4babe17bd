// Host side of the QuantWM 2-bit KV cache library: argument checks, arena
// layout, the epoch directory, split-KV planning and kernel launches.
// Every public entry point is declared (and documented) in include/qwm.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include <mutex>

#include "qwm.h"
#include "qwm_internal.h"

// Scratch of qwm_attend_noalloc: the q . U_r table, the decode path's q . C
// table and the split-KV partials of one call, in a fixed device array
// (64 MiB on every device the library runs on, held until the process
// ends) instead of the caller's arena. In host code `scratch` names a host
// stand-in; its device address, resolved once per device, is what kernels
// receive.
static constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

qwm_status fail(qwm_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

qwm_status fail_hip(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return QWM_ERR_HIP;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
  size_t kcode, vcode, kparam, vparam, ids, coef;
  size_t epochC, epochS, epochU, C32, kmC32, U64, gram, diag, build_ids, km_perm, km_off, km_woff, km_ccd, qU, qc,
      part_o, part_ml, work, qpart;
  size_t total;
  int64_t capP, part_rows;
};

qwm_status check_desc(const qwm_desc* d) {
  if (!d) return fail(QWM_ERR_INVALID_ARG, "desc is NULL");
  if (d->heads < 1) return fail(QWM_ERR_INVALID_ARG, "heads must be >= 1");
  if (d->dtype != QWM_BF16 && d->dtype != QWM_F32) return fail(QWM_ERR_INVALID_ARG, "dtype must be QWM_BF16 or QWM_F32");
  if (d->objective != QWM_OBJ_QSAC && d->objective != QWM_OBJ_NEAREST && d->objective != QWM_OBJ_POSTQ)
    return fail(QWM_ERR_INVALID_ARG, "objective must be QWM_OBJ_QSAC, QWM_OBJ_NEAREST or QWM_OBJ_POSTQ");
  if (d->capacity_tokens < 1) return fail(QWM_ERR_INVALID_ARG, "capacity_tokens must be >= 1");
  if (d->max_query_tokens < 1) return fail(QWM_ERR_INVALID_ARG, "max_query_tokens must be >= 1");
  if (d->max_build_tokens < 1) return fail(QWM_ERR_INVALID_ARG, "max_build_tokens must be >= 1");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(QWM_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->group != qwm::kGroup) return fail(QWM_ERR_UNSUPPORTED, "group must be 32");
  if (d->n_centroids < 1 || d->n_centroids > 256) return fail(QWM_ERR_UNSUPPORTED, "n_centroids must be 1..256");
  if (d->rank < 0 || d->rank > qwm::kRankPad) return fail(QWM_ERR_UNSUPPORTED, "rank must be 0..16");
  if (d->max_epochs < 1 || d->max_epochs > qwm::kMaxEpochs) return fail(QWM_ERR_UNSUPPORTED, "max_epochs must be 1..64");
  if (d->capacity_tokens > ((int64_t)1 << 26))
    return fail(QWM_ERR_UNSUPPORTED, "capacity_tokens beyond 2^26 per head");
  if (d->max_query_tokens > (int64_t)INT32_MAX / 2) return fail(QWM_ERR_UNSUPPORTED, "max_query_tokens too large");
  if (d->max_build_tokens > ((int64_t)1 << 22)) return fail(QWM_ERR_UNSUPPORTED, "max_build_tokens beyond 2^22");
  return QWM_OK;
}

// Bytes one token of one head occupies in the record regions (K codes, V
// codes, K params, V params, id, coefficients), and one epoch slot of one
// head in the calibration regions (C, S, U). make_layout sizes the regions
// from these, and qwm_storage_bytes reports them.
int64_t token_record_bytes(const qwm_desc* d) {
  const int64_t D = d->head_dim, nG = D / qwm::kGroup;
  return D / 4 + D / 4 + nG * 4 + nG * 4 + 1 + (int64_t)d->rank * 2;
}
int64_t epoch_table_bytes(const qwm_desc* d) {
  const int64_t D = d->head_dim, nG = D / qwm::kGroup, esz = d->dtype == QWM_BF16 ? 2 : 4;
  return (int64_t)d->n_centroids * D * esz + nG * 4 + D * (int64_t)d->rank * 4;
}

Layout make_layout(const qwm_desc* d) {
  Layout L{};
  const int64_t H = d->heads, D = d->head_dim, nG = D / qwm::kGroup, m = d->n_centroids, r = d->rank;
  const int64_t E = d->max_epochs, esz = d->dtype == QWM_BF16 ? 2 : 4;
  const int64_t maxq = d->max_query_tokens;
  L.capP = (d->capacity_tokens + qwm::kTileKV - 1) / qwm::kTileKV * qwm::kTileKV;
  const int64_t big = 1 << 18;
  int64_t pr = 8 * H * maxq > big ? 8 * H * maxq : big;
  if (pr > 16 * H * maxq) pr = 16 * H * maxq;
  // decode-shaped calls split the cache more finely (up to 64 ways)
  const int64_t dq = maxq < qwm::kDecodeMaxQ ? maxq : qwm::kDecodeMaxQ;
  if (pr < 64 * H * dq) pr = 64 * H * dq;
  L.part_rows = pr;
  const int64_t nqp_max = (dq + qwm::kDecodeQ - 1) / qwm::kDecodeQ * qwm::kDecodeQ;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.kcode = take((size_t)(H * L.capP * D / 4));
  L.vcode = take((size_t)(H * L.capP * D / 4));
  L.kparam = take((size_t)(H * L.capP * nG * 4));
  L.vparam = take((size_t)(H * L.capP * nG * 4));
  L.ids = take((size_t)(H * L.capP));
  // the attention tile loads read 16 coefficient halves per token whatever r
  // is (those past r are discarded), hence the tail
  L.coef = take((size_t)(H * L.capP * r * 2 + 64));
  // (the record regions hold token_record_bytes per token-head)
  L.epochC = take((size_t)((E + 1) * H * m * D * esz));
  L.epochS = take((size_t)((E + 1) * H * nG * 4));
  L.epochU = take((size_t)((E + 1) * H * D * r * 4));
  // (each epoch slot holds epoch_table_bytes per head)
  L.C32 = take((size_t)(H * m * D * 4));
  L.kmC32 = take((size_t)(H * m * D * 4));
  L.U64 = take((size_t)(H * D * r * 8));
  L.gram = take((size_t)(H * qwm::kGramMaxChunks * D * D * 8));
  L.diag = take((size_t)(H * qwm::kGramMaxChunks * D * 8));
  L.build_ids = take((size_t)(H * d->max_build_tokens));
  L.km_perm = take((size_t)(H * d->max_build_tokens * 4));
  L.km_off = take((size_t)(H * 257 * 4));
  L.km_woff = take((size_t)(H * 257 * 4));
  // centroid-to-centroid bounds of the pruned assignment (128 or more centroids)
  L.km_ccd = take(m >= 128 ? (size_t)(H * m * m * 4) : 0);
  L.qU = take((size_t)(H * E * maxq * qwm::kRankPad * 4));
  // the decode path's q . C tables; the bf16 head_dim-128 prefill path keeps
  // an fp16 copy of the epochs' centroid tables in the same region
  const int64_t qc_bytes = H * E * m * nqp_max * 4;
  const int64_t c16_bytes = (d->dtype == QWM_BF16 && D == 128) ? H * E * m * D * 2 : 0;
  L.qc = take((size_t)(qc_bytes > c16_bytes ? qc_bytes : c16_bytes));
  L.part_o = take((size_t)(pr * D * 4));
  L.part_ml = take((size_t)(pr * 2 * 4));
  L.work = take(sizeof(unsigned long long) * QWM_K_COUNT);  // profiling work counters
  // per-half best (J, id) of split centroid scans (k-means on few Keys)
  L.qpart = take((size_t)(2 * H * qwm::kQuantSplitMaxTokens * 8));
  L.total = off;
  return L;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of `scratch` on device `dev`, which must be current:
// hipGetSymbolAddress on first use per device, then the kept pointer.
qwm_status static_scratch(int dev, uint8_t** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(QWM_ERR_HIP, "no device for the static scratch");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail_hip(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch address");
    g_scratch_dev[dev] = reinterpret_cast<uint8_t*>(p);
  }
  *out = g_scratch_dev[dev];
  return QWM_OK;
}

struct DeviceGuard {
  int prev = -1, dev;
  explicit DeviceGuard(int d) : dev(d) {
    if (dev < 0) return;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    if (prev >= 0 && prev != dev) (void)hipSetDevice(prev);
  }
};

struct ProfRec {
  int kid;
  hipEvent_t a, b;
};

}  // namespace

struct qwm_cache {
  qwm_desc desc{};
  Layout L{};
  int H = 0, D = 0, nG = 0, m = 0, r = 0, dtype = 0, esz = 0;
  int device = 0;
  int ncu = 256;  // compute units of the device
  hipStream_t stream = nullptr;
  uint8_t* arena = nullptr;
  qwm::CacheView view{};
  int64_t length = 0;
  std::vector<int64_t> epoch_start;  // committed epoch i lives in slot i
  bool staged_subspace = false;
  int obj = 0;  // qwm::kObjQsac or qwm::kObjNearest
  // The eigensolve of build_subspace runs on `side` (created on first use,
  // default priority) so the k-means of build_centroids, which needs only the
  // sensitivity, overlaps it; `stream` waits for `join_ev` before the staged
  // U is read or the Gram buffer is written again. The eigensolve reads
  // arena memory only, never a caller buffer.
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
  bool side_pending = false;
  bool profile = false;
  std::vector<ProfRec> pending;
  double prof_ms[QWM_K_COUNT] = {};
  int64_t prof_n[QWM_K_COUNT] = {};
  // channel evaluations of the centroid rule while profiling: full passes are
  // counted here, the pruned assignment counts its own in the arena's `work`
  // counters, cleared before its first launch after profiling was enabled
  double work_host[QWM_K_COUNT] = {};
  bool work_clear = true;

  uint8_t* slotC(int slot) const {
    return arena + L.epochC + (size_t)slot * H * m * D * esz;
  }
  float* slotS(int slot) const {
    return reinterpret_cast<float*>(arena + L.epochS) + (size_t)slot * H * nG;
  }
  float* slotU(int slot) const {
    return reinterpret_cast<float*>(arena + L.epochU) + (size_t)slot * H * D * r;
  }
  int staged() const { return desc.max_epochs; }
  float* C32() const { return reinterpret_cast<float*>(arena + L.C32); }
  float* kmC32() const { return reinterpret_cast<float*>(arena + L.kmC32); }
  double* U64() const { return reinterpret_cast<double*>(arena + L.U64); }
  double* gram() const { return reinterpret_cast<double*>(arena + L.gram); }
  double* diag() const { return reinterpret_cast<double*>(arena + L.diag); }
  uint8_t* build_ids() const { return arena + L.build_ids; }
  int32_t* km_perm() const { return reinterpret_cast<int32_t*>(arena + L.km_perm); }
  int32_t* km_off() const { return reinterpret_cast<int32_t*>(arena + L.km_off); }
  int32_t* km_woff() const { return reinterpret_cast<int32_t*>(arena + L.km_woff); }
  float* km_ccd() const { return reinterpret_cast<float*>(arena + L.km_ccd); }
  float* qU() const { return reinterpret_cast<float*>(arena + L.qU); }
  float* qc() const { return reinterpret_cast<float*>(arena + L.qc); }
  float* part_o() const { return reinterpret_cast<float*>(arena + L.part_o); }
  float* part_ml() const { return reinterpret_cast<float*>(arena + L.part_ml); }
  unsigned long long* work() const { return reinterpret_cast<unsigned long long*>(arena + L.work); }
  // The split scan buffer when an n-token k-means assignment pass should
  // scan its centroids in two halves, else null. A workgroup's time is set
  // by its own dependency chains, not by how busy its CU is, so a pass of B
  // blocks over R resident ones takes ceil(B / R) full rounds; split, it
  // takes ceil(2B / R) half rounds plus a short finishing pass. Split when
  // that is fewer (the streaming refresh's 1,560 Keys of 40 heads: 1,000
  // blocks, 768 resident, 3 half rounds against 2 full ones; 157 -> 143 us
  // per pass).
  uint2* quant_split(int64_t n) const {
    if (n > qwm::kQuantSplitMaxTokens) return nullptr;
    const int64_t B = (n + 63) / 64 * H, R = (int64_t)qwm::kQuantBlocksPerCU * ncu;
    const int64_t full = (B + R - 1) / R, halves = (2 * B + R - 1) / R;
    return halves < 2 * full ? reinterpret_cast<uint2*>(arena + L.qpart) : nullptr;
  }
  // the pruned assignment's counter while profiling (cleared on first use), else null
  unsigned long long* work_counter(int kid) {
    if (!profile || no_events) return nullptr;
    if (work_clear) {
      if (qwm::launch_fill(reinterpret_cast<float*>(work()), 2 * QWM_K_COUNT, 0.0f, stream) != hipSuccess)
        return nullptr;
      work_clear = false;
    }
    return work() + kid;
  }
  void count_full_pass(int kid, int64_t n) {
    if (profile && !no_events) work_host[kid] += (double)H * (double)n * m * D;
  }

  // Launch wrapper: optional event timing around one launch on stream `s`.
  bool no_events = false;  // set by qwm_attend_noalloc: record no timing events
  template <class F>
  hipError_t run_on(hipStream_t s, int kid, F&& f) {
    hipEvent_t a = nullptr, b = nullptr;
    const bool timed = profile && !no_events;
    if (timed) {
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return hipErrorOutOfMemory;
      (void)hipEventRecord(a, s);
    }
    hipError_t e = f();
    if (timed) {
      (void)hipEventRecord(b, s);
      pending.push_back({kid, a, b});
    }
    return e;
  }
  template <class F>
  hipError_t run(int kid, F&& f) {
    return run_on(stream, kid, f);
  }
  // Make the cache stream wait for an eigensolve still running on `side`.
  hipError_t join_side() {
    if (!side_pending) return hipSuccess;
    side_pending = false;
    return hipStreamWaitEvent(stream, join_ev, 0);
  }
};

namespace {

qwm_status check_cache(const qwm_cache* c) {
  if (!c) return fail(QWM_ERR_INVALID_ARG, "cache is NULL");
  return QWM_OK;
}

qwm_status need_device(const qwm_cache* c) {
  if (c->device < 0) return fail(QWM_ERR_HIP, "no HIP device was available when the cache was created");
  return QWM_OK;
}

qwm_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(QWM_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(QWM_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned");
  return QWM_OK;
}

// Commit the staged calibration as a new epoch (or in place of an epoch that
// holds no token yet). Capacity was checked by the caller.
qwm_status commit_staged(qwm_cache* c) {
  hipError_t je = c->join_side();
  if (je != hipSuccess) return fail_hip(je, "join eigensolve");
  int slot = (int)c->epoch_start.size();
  if (!c->epoch_start.empty() && c->epoch_start.back() == c->length) slot -= 1;
  const int st = c->staged();
  hipError_t e = c->run(QWM_K_OTHER, [&] {
    return qwm::launch_commit(c->D, c->dtype, c->slotC(st), c->slotS(st), c->slotU(st), c->slotC(slot), c->slotS(slot),
                              c->slotU(slot), c->H, c->m, c->r, c->C32(), c->U64(), c->stream);
  });
  if (e != hipSuccess) return fail_hip(e, "commit");
  if (slot == (int)c->epoch_start.size())
    c->epoch_start.push_back(c->length);
  else
    c->epoch_start[slot] = c->length;
  c->staged_subspace = false;
  return QWM_OK;
}

bool epoch_room(const qwm_cache* c) {
  if (!c->epoch_start.empty() && c->epoch_start.back() == c->length) return true;  // replaces an empty epoch
  return (int)c->epoch_start.size() < c->desc.max_epochs;
}

// Segments of the cache (one per epoch holding tokens) plus the self segment.
void make_plan(const qwm_cache* c, int64_t nself, bool with_self, qwm::AttnPlan& p) {
  std::memset(&p, 0, sizeof(p));
  int n = 0;
  const int E = (int)c->epoch_start.size();
  for (int e = 0; e < E; ++e) {
    const int64_t s = c->epoch_start[e];
    const int64_t t = (e + 1 < E) ? c->epoch_start[e + 1] : c->length;
    if (t > s) {
      p.seg_start[n] = (int32_t)s;
      p.seg_len[n] = (int32_t)(t - s);
      p.seg_epoch[n] = e;
      ++n;
    }
  }
  if (with_self && nself > 0) {
    p.seg_start[n] = 0;
    p.seg_len[n] = (int32_t)nself;
    p.seg_epoch[n] = -1;
    ++n;
  }
  p.n_seg = n;
  p.tile_prefix[0] = 0;
  for (int i = 0; i < n; ++i)
    p.tile_prefix[i + 1] = p.tile_prefix[i] + (p.seg_len[i] + qwm::kTileKV - 1) / qwm::kTileKV;
}

// Per-call scratch of the attention paths: the q . U_r table [H][E][n_q][16],
// the decode path's q . C table [H][E][m][nqp] and the split-KV partials
// (part_rows rows of D floats in part_o, (max, sum) pairs in part_ml). Every
// entry a call reads is written by that call first.
struct AttnWork {
  float* qU;
  float* qc;
  float* part_o;
  float* part_ml;
  int64_t part_rows;
  void* c16;  // room for the fp16 centroid copy of the bf16 head_dim-128 prefill path, or null
};

AttnWork arena_work(const qwm_cache* c) {
  // the arena's q . C region is sized to hold the copy (make_layout)
  void* c16 = (c->dtype == QWM_BF16 && c->D == 128) ? static_cast<void*>(c->qc()) : nullptr;
  return {c->qU(), c->qc(), c->part_o(), c->part_ml(), c->L.part_rows, c16};
}

qwm::AttnArgs base_args(qwm_cache* c, const AttnWork& w) {
  qwm::AttnArgs a{};
  a.cache = c->view;
  a.Cbase = c->slotC(0);
  a.epoch_C_stride = (int64_t)c->H * c->m * c->D * c->esz;
  a.H = c->H;
  a.m = c->m;
  a.r = c->r;
  a.part_o = w.part_o;
  a.part_ml = w.part_ml;
  return a;
}

// Queries per attention workgroup: the fewest workgroups of at most 256
// Queries, with the 32-Query waves spread evenly over them (880 Queries: 4 x
// 224 rather than 3 x 256 + 112), so no workgroup carries more live waves
// than it must.
int queries_per_block(int64_t n_q) {
  if (n_q < 1) return qwm::kTileQ;
  const int64_t nblk = (n_q + qwm::kTileQ - 1) / qwm::kTileQ;
  const int64_t waves = (n_q + 31) / 32;
  return (int)(32 * ((waves + nblk - 1) / nblk));
}

// Split the KV tiles so that the workgroups fill the device in as few
// rounds as possible: cost = rounds x (tiles per workgroup + 2 for its
// prologue and epilogue) + 2 for the merge pass when split; one workgroup
// per CU for head_dim 128 (their LDS stages take most of the CU's 160 KB).
int choose_splits(const qwm_cache* c, int64_t n_q, int T, int64_t part_rows) {
  const int64_t qtiles = (n_q + qwm::kTileQ - 1) / qwm::kTileQ;
  const int64_t slots = (int64_t)c->ncu * (c->D == 128 ? 1 : 2);
  int64_t splits = 1, best = -1;
  for (int64_t sp = 1; sp <= 16 && sp <= T; ++sp) {
    if (sp > 1 && sp * c->H * n_q > part_rows) break;
    const int64_t rounds = (qtiles * c->H * sp + slots - 1) / slots;
    const int64_t cost = rounds * ((T + sp - 1) / sp + 2) + (sp > 1 ? 2 : 0);
    if (best < 0 || cost < best) {
      best = cost;
      splits = sp;
    }
  }
  return (int)splits;
}

// The decode path of qwm_attend: q . U_r and q . C tables, then the decode
// kernel over splits of the tiles and the log-sum-exp merge.
bool use_decode(const qwm_cache* c, int32_t mask, int64_t n_q) {
  return c->dtype == QWM_BF16 && c->D == 128 && mask == QWM_SELF_NONE && n_q <= qwm::kDecodeMaxQ && (c->r % 2) == 0;
}

qwm_status attend_decode(qwm_cache* c, const void* q, int64_t n_q, float softmax_scale, float* out,
                         const qwm::AttnPlan& p, const AttnWork& w) {
  const int T = p.tile_prefix[p.n_seg];
  const int E = (int)c->epoch_start.size();
  const int64_t qtiles = (n_q + qwm::kDecodeQ - 1) / qwm::kDecodeQ;
  const int nqp = (int)(qtiles * qwm::kDecodeQ);
  // as many single-wave workgroups as the CUs hold at once (one round: a
  // workgroup past that would start when the first round ends), at least 4
  // tiles per split
  int64_t splits = (int64_t)qwm::kDecodeWavesPerCU * c->ncu / (qtiles * c->H);
  if (splits < 1) splits = 1;
  const int64_t cap = T / 4 > 1 ? T / 4 : 1;
  if (splits > cap) splits = cap;
  if (splits > 64) splits = 64;
  while (splits > 1 && splits * c->H * n_q > w.part_rows) --splits;
  qwm::DecodeArgs d{};
  d.q = q;
  d.qc = w.qc;
  d.qU = w.qU;
  d.cache = c->view;
  d.nq = n_q;
  d.nqp = nqp;
  d.H = c->H;
  d.m = c->m;
  d.r = c->r;
  d.E = E;
  d.scale_log2 = softmax_scale * 1.4426950408889634f;
  d.splits = (int)splits;
  d.out = out;
  d.part_o = w.part_o;
  d.part_ml = w.part_ml;
  hipError_t e = hipSuccess;
  if (c->r > 0) {
    e = c->run(QWM_K_QU, [&] {
      return qwm::launch_qu(c->D, c->dtype, q, n_q, c->H, c->r, c->slotU(0), (int64_t)c->H * c->D * c->r, E, w.qU,
                            c->stream);
    });
    if (e != hipSuccess) return fail_hip(e, "qU");
  }
  e = c->run(QWM_K_QU, [&] {
    return qwm::launch_qc(q, n_q, nqp, c->slotC(0), (int64_t)c->H * c->m * c->D, c->H, c->m, E,
                          softmax_scale < 0.0f ? -1.0f : 1.0f, w.qc, c->stream);
  });
  if (e != hipSuccess) return fail_hip(e, "qC");
  e = c->run(QWM_K_ATTEND, [&] { return qwm::launch_decode(d, p, c->stream); });
  if (e != hipSuccess) return fail_hip(e, "decode");
  if (splits > 1) {
    qwm::AttnArgs a = base_args(c, w);
    a.nq = n_q;
    a.splits = (int)splits;
    a.out = out;
    e = c->run(QWM_K_MERGE, [&] { return qwm::launch_merge(c->D, a, c->stream); });
    if (e != hipSuccess) return fail_hip(e, "merge");
  }
  return QWM_OK;
}

// Argument and state checks shared by qwm_attend and qwm_attend_noalloc,
// which differ in the bound on n_q (max_query_tokens; for the static scratch
// 2^24 here and the size of its tables later).
qwm_status check_attend(qwm_cache* c, const void* q, int64_t n_q, const void* k_self, const void* v_self,
                        int64_t n_self, int32_t mask, float softmax_scale, float* out, bool arena_scratch) {
  qwm_status st;
  if ((st = check_cache(c)) != QWM_OK) return st;
  if ((st = check_ptr(q, "q")) != QWM_OK) return st;
  if ((st = check_ptr(out, "out")) != QWM_OK) return st;
  if (n_q < 1) return fail(QWM_ERR_INVALID_ARG, "n_q must be >= 1");
  if (arena_scratch && n_q > c->desc.max_query_tokens) return fail(QWM_ERR_CAPACITY, "n_q exceeds max_query_tokens");
  if (n_q > ((int64_t)1 << 24)) return fail(QWM_ERR_CAPACITY, "n_q beyond 2^24");
  if (mask != QWM_SELF_NONE && mask != QWM_SELF_FULL && mask != QWM_SELF_CAUSAL)
    return fail(QWM_ERR_INVALID_ARG, "bad mask");
  if (!std::isfinite(softmax_scale) || softmax_scale == 0.0f)
    return fail(QWM_ERR_INVALID_ARG, "softmax_scale must be finite and nonzero");
  if (mask == QWM_SELF_NONE) {
    if (n_self != 0) return fail(QWM_ERR_INVALID_ARG, "n_self must be 0 with QWM_SELF_NONE");
  } else {
    if (n_self < 1) return fail(QWM_ERR_INVALID_ARG, "a self mask needs n_self >= 1");
    if (n_self > ((int64_t)1 << 22)) return fail(QWM_ERR_CAPACITY, "n_self beyond 2^22");
    if ((st = check_ptr(k_self, "k_self")) != QWM_OK) return st;
    if ((st = check_ptr(v_self, "v_self")) != QWM_OK) return st;
    if (mask == QWM_SELF_CAUSAL && n_self != n_q) return fail(QWM_ERR_INVALID_ARG, "causal self needs n_self == n_q");
  }
  if (c->epoch_start.empty()) return fail(QWM_ERR_STATE, "attend before a committed epoch");
  if (c->length == 0 && mask == QWM_SELF_NONE) return fail(QWM_ERR_STATE, "nothing to attend to");
  return need_device(c);
}

// The attention of qwm_attend with its scratch in `w` (device current).
qwm_status attend_impl(qwm_cache* c, const void* q, int64_t n_q, const void* k_self, const void* v_self,
                       int64_t n_self, int32_t mask, float softmax_scale, float* out, const AttnWork& w) {
  qwm::AttnPlan p;
  make_plan(c, n_self, mask != QWM_SELF_NONE, p);
  const int T = p.tile_prefix[p.n_seg];
  const int E = (int)c->epoch_start.size();
  qwm::AttnArgs a = base_args(c, w);
  a.q = q;
  a.qU = w.qU;
  a.kself = k_self;
  a.vself = v_self;
  a.nq = n_q;
  a.nself = n_self;
  a.causal_self = (mask == QWM_SELF_CAUSAL) ? 1 : 0;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.n_epoch_slots = E;
  a.qpb = queries_per_block(n_q);
  a.out = out;
  a.C16 = w.c16;
  // Few Queries over bf16 Keys: the decode kernel (2-bit codes as the MFMA
  // operand, one wave per workgroup, many splits)
  if (use_decode(c, mask, n_q)) return attend_decode(c, q, n_q, softmax_scale, out, p, w);
  a.splits = choose_splits(c, n_q, T, w.part_rows);
  hipError_t e = hipSuccess;
  if (c->r > 0) {  // the kernels read no qU at rank 0
    e = c->run(QWM_K_QU, [&] {
      return qwm::launch_qu(c->D, c->dtype, q, n_q, c->H, c->r, c->slotU(0), (int64_t)c->H * c->D * c->r, E, w.qU,
                            c->stream);
    });
    if (e != hipSuccess) return fail_hip(e, "qU");
  }
  e = c->run(QWM_K_ATTEND, [&] { return qwm::launch_attend(c->D, c->dtype, a, p, c->stream); });
  if (e != hipSuccess) return fail_hip(e, "attend");
  if (a.splits > 1) {
    e = c->run(QWM_K_MERGE, [&] { return qwm::launch_merge(c->D, a, c->stream); });
    if (e != hipSuccess) return fail_hip(e, "merge");
  }
  return QWM_OK;
}

}  // namespace

extern "C" {

const char* qwm_last_error(void) { return g_last_error.c_str(); }
#ifndef QWM_SOURCE_HASH
#define QWM_SOURCE_HASH "unstamped"
#endif
// "qwm <version> gfx950 src:<hash>": the hash covers every source file of the
// library (video_world_model_amd/build.py computes and stamps it).
const char* qwm_version(void) { return "qwm 0.2 gfx950 src:" QWM_SOURCE_HASH; }

qwm_status qwm_arena_bytes(const qwm_desc* desc, size_t* bytes) {
  qwm_status st = check_desc(desc);
  if (st != QWM_OK) return st;
  if (!bytes) return fail(QWM_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = make_layout(desc).total;
  return QWM_OK;
}

qwm_status qwm_storage_bytes(const qwm_desc* desc, int64_t n_tokens, int32_t n_epochs, size_t* record_bytes,
                             size_t* table_bytes) {
  qwm_status st = check_desc(desc);
  if (st != QWM_OK) return st;
  if (!record_bytes || !table_bytes) return fail(QWM_ERR_INVALID_ARG, "NULL argument");
  if (n_tokens < 0 || n_tokens > desc->capacity_tokens)
    return fail(QWM_ERR_INVALID_ARG, "n_tokens must be in [0, capacity_tokens]");
  if (n_epochs < 0 || n_epochs > desc->max_epochs) return fail(QWM_ERR_INVALID_ARG, "n_epochs must be in [0, max_epochs]");
  *record_bytes = (size_t)desc->heads * (size_t)n_tokens * (size_t)token_record_bytes(desc);
  *table_bytes = (size_t)n_epochs * (size_t)desc->heads * (size_t)epoch_table_bytes(desc);
  return QWM_OK;
}

qwm_status qwm_create(const qwm_desc* desc, void* dev_arena, size_t arena_bytes, void* stream, qwm_cache** out) {
  qwm_status st = check_desc(desc);
  if (st != QWM_OK) return st;
  if (!out) return fail(QWM_ERR_INVALID_ARG, "out is NULL");
  if (!dev_arena) return fail(QWM_ERR_INVALID_ARG, "dev_arena is NULL");
  const Layout L = make_layout(desc);
  if ((reinterpret_cast<uintptr_t>(dev_arena) % kAlign) != 0)
    return fail(QWM_ERR_ARENA_TOO_SMALL, "dev_arena must be 256-byte aligned");
  if (arena_bytes < L.total)
    return fail(QWM_ERR_ARENA_TOO_SMALL, "arena has " + std::to_string(arena_bytes) + " bytes, needs " +
                                             std::to_string(L.total));
  // Without a usable HIP device the handle still exists (device -1) so that
  // every argument and state check can run; calls that would enqueue work
  // then fail with QWM_ERR_HIP after their checks.
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  qwm_cache* c = new qwm_cache();
  c->desc = *desc;
  c->L = L;
  c->H = desc->heads;
  c->D = desc->head_dim;
  c->nG = desc->head_dim / qwm::kGroup;
  c->m = desc->n_centroids;
  c->r = desc->rank;
  c->obj = desc->objective == QWM_OBJ_NEAREST ? qwm::kObjNearest
           : desc->objective == QWM_OBJ_POSTQ ? qwm::kObjPostq
                                              : qwm::kObjQsac;
  c->dtype = desc->dtype;
  c->esz = desc->dtype == QWM_BF16 ? 2 : 4;
  c->device = dev;
  if (dev >= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) c->ncu = n;
    // set-up of qwm_attend_noalloc on this (current) device
    uint8_t* sp = nullptr;
    if ((st = static_scratch(dev, &sp)) != QWM_OK) {
      delete c;
      return st;
    }
  }
  c->stream = reinterpret_cast<hipStream_t>(stream);
  c->arena = reinterpret_cast<uint8_t*>(dev_arena);
  c->view.kcode = c->arena + L.kcode;
  c->view.vcode = c->arena + L.vcode;
  c->view.kparam = reinterpret_cast<uint32_t*>(c->arena + L.kparam);
  c->view.vparam = reinterpret_cast<uint32_t*>(c->arena + L.vparam);
  c->view.ids = c->arena + L.ids;
  c->view.coef = reinterpret_cast<uint16_t*>(c->arena + L.coef);
  c->view.capP = L.capP;
  *out = c;
  return QWM_OK;
}

qwm_status qwm_destroy(qwm_cache* c) {
  if (!c) return fail(QWM_ERR_INVALID_ARG, "cache is NULL");
  if (c->side) {
    DeviceGuard g(c->device);
    (void)hipStreamSynchronize(c->side);
    (void)hipEventDestroy(c->fork_ev);
    (void)hipEventDestroy(c->join_ev);
    (void)hipStreamDestroy(c->side);
  }
  for (auto& rec : c->pending) {
    (void)hipEventDestroy(rec.a);
    (void)hipEventDestroy(rec.b);
  }
  delete c;
  return QWM_OK;
}

qwm_status qwm_build_subspace(qwm_cache* c, const void* q_hist, int64_t n_hist) {
  qwm_status st;
  if ((st = check_cache(c)) != QWM_OK) return st;
  if ((st = check_ptr(q_hist, "q_hist")) != QWM_OK) return st;
  if (n_hist < 1) return fail(QWM_ERR_INVALID_ARG, "n_hist must be >= 1");
  if (n_hist > (int64_t)INT32_MAX / 2) return fail(QWM_ERR_CAPACITY, "n_hist too large");
  if ((st = need_device(c)) != QWM_OK) return st;
  DeviceGuard g(c->device);
  hipError_t e;
  if (!c->side) {
    if ((e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking)) != hipSuccess) {
      c->side = nullptr;
      return fail_hip(e, "create eigensolve stream");
    }
    if ((e = hipEventCreateWithFlags(&c->fork_ev, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&c->join_ev, hipEventDisableTiming)) != hipSuccess)
      return fail_hip(e, "create eigensolve events");
  }
  // the previous eigensolve may still read the Gram buffer
  if ((e = c->join_side()) != hipSuccess) return fail_hip(e, "join eigensolve");
  const int st_slot = c->staged();
  const int nchunk = qwm::gram_chunks(n_hist);
  // Every read of q_hist stays on the cache stream (the caller may release
  // it once that stream has passed this call): the Gram diagonal and the
  // sensitivity, then the full Gram. Only the eigensolve, which reads arena
  // memory alone, runs on `side`, overlapping the k-means that follows.
  e = c->run(QWM_K_GRAM, [&] {
    return qwm::launch_diag(c->D, c->dtype, q_hist, n_hist, c->H, c->diag(), c->stream);
  });
  if (e != hipSuccess) return fail_hip(e, "gram diagonal");
  e = c->run(QWM_K_GRAM, [&] {
    return qwm::launch_sens(c->D, c->diag(), nchunk, n_hist, c->H, c->slotS(st_slot), c->stream);
  });
  if (e != hipSuccess) return fail_hip(e, "sensitivity");
  if (c->r == 0) {  // PSAC off: no basis to compute
    c->staged_subspace = true;
    return QWM_OK;
  }
  e = c->run(QWM_K_GRAM, [&] {
    return qwm::launch_gram(c->D, c->dtype, q_hist, n_hist, c->H, c->gram(), c->stream);
  });
  if (e != hipSuccess) return fail_hip(e, "gram");
  if ((e = hipEventRecord(c->fork_ev, c->stream)) != hipSuccess) return fail_hip(e, "fork eigensolve");
  if ((e = hipStreamWaitEvent(c->side, c->fork_ev, 0)) != hipSuccess) return fail_hip(e, "fork eigensolve");
  e = c->run_on(c->side, QWM_K_EIGEN, [&] {
    return qwm::launch_eigen(c->D, c->gram(), nchunk, c->H, c->r, c->slotU(st_slot), c->side);
  });
  if (e != hipSuccess) return fail_hip(e, "eigen");
  if ((e = hipEventRecord(c->join_ev, c->side)) != hipSuccess) return fail_hip(e, "join eigensolve");
  c->side_pending = true;
  c->staged_subspace = true;
  return QWM_OK;
}

qwm_status qwm_build_centroids(qwm_cache* c, const void* keys, int64_t n_keys, int32_t iters) {
  qwm_status st;
  if ((st = check_cache(c)) != QWM_OK) return st;
  if ((st = check_ptr(keys, "keys")) != QWM_OK) return st;
  if (n_keys < 1) return fail(QWM_ERR_INVALID_ARG, "n_keys must be >= 1");
  if (iters < 0) return fail(QWM_ERR_INVALID_ARG, "iters must be >= 0");
  if (n_keys > c->desc.max_build_tokens) return fail(QWM_ERR_CAPACITY, "n_keys exceeds max_build_tokens");
  // The nearest-centroid rule with PSAC off needs no historical Queries: the
  // staged sensitivity is then all zeros.
  const bool no_subspace_needed = (c->obj == qwm::kObjNearest && c->r == 0);
  if (!c->staged_subspace && !no_subspace_needed)
    return fail(QWM_ERR_STATE, "build_centroids needs build_subspace first");
  if (!epoch_room(c)) return fail(QWM_ERR_CAPACITY, "max_epochs reached");
  if ((st = need_device(c)) != QWM_OK) return st;
  DeviceGuard g(c->device);
  const int stg = c->staged();
  hipError_t e;
  if (!c->staged_subspace) {
    e = c->run(QWM_K_OTHER, [&] { return qwm::launch_fill(c->slotS(stg), (int64_t)c->H * c->nG, 0.0f, c->stream); });
    if (e != hipSuccess) return fail_hip(e, "zero sensitivity");
  }
  e = c->run(QWM_K_OTHER, [&] {
    return qwm::launch_kmeans_seed(c->D, c->dtype, keys, n_keys, c->H, c->m, c->slotC(stg), c->kmC32(), c->stream);
  });
  if (e != hipSuccess) return fail_hip(e, "kmeans seed");
  for (int it = 0; it < iters; ++it) {
    // Pruning pays for its grouping pass only with many centroids (below 128
    // the skipped work does not cover the bound computations and the
    // serialized candidate loads) that each hold enough Keys to fill waves of
    // 64 (a wave serves the Keys of one previous centroid).
    // (The post-rounding error is no seminorm: it always takes the full pass.)
    if (it == 0 || c->m < 128 || n_keys < 32 * (int64_t)c->m || c->obj == qwm::kObjPostq) {
      qwm::QuantArgs a{};
      a.k = keys;
      a.v = nullptr;
      a.n = n_keys;
      a.C32 = c->kmC32();
      a.S = c->slotS(stg);
      a.ids_out = c->build_ids();
      a.H = c->H;
      a.m = c->m;
      a.r = c->r;
      a.obj = c->obj;
      a.part = c->quant_split(n_keys);
      e = c->run(QWM_K_ASSIGN, [&] { return qwm::launch_quantize(c->D, c->dtype, a, c->stream); });
      if (e != hipSuccess) return fail_hip(e, "kmeans assign");
      c->count_full_pass(QWM_K_ASSIGN, n_keys);
    } else {  // the same ids, skipping candidates the triangle inequality rules out
      e = c->run(QWM_K_OTHER, [&] {
        return qwm::launch_kmeans_ccd(c->D, c->obj, c->H, c->m, c->kmC32(), c->slotS(stg), c->km_ccd(), c->stream);
      });
      if (e != hipSuccess) return fail_hip(e, "kmeans centroid distances");
      e = c->run(QWM_K_OTHER, [&] {
        return qwm::launch_kmeans_bucket(c->build_ids(), n_keys, c->H, c->m, c->km_perm(), c->km_off(), c->km_woff(),
                                         c->stream);
      });
      if (e != hipSuccess) return fail_hip(e, "kmeans bucket");
      unsigned long long* work = c->work_counter(QWM_K_ASSIGN);
      e = c->run(QWM_K_ASSIGN, [&] {
        return qwm::launch_kmeans_assign_pruned(c->D, c->dtype, c->obj, keys, n_keys, c->H, c->m, c->kmC32(), c->slotS(stg),
                                                c->km_perm(), c->km_off(), c->km_woff(), c->km_ccd(), c->build_ids(),
                                                work, c->stream);
      });
      if (e != hipSuccess) return fail_hip(e, "kmeans assign");
    }
    e = c->run(QWM_K_UPDATE, [&] {
      return qwm::launch_kmeans_update(c->D, c->dtype, keys, c->build_ids(), n_keys, c->H, c->m, c->slotC(stg),
                                       c->kmC32(), c->stream);
    });
    if (e != hipSuccess) return fail_hip(e, "kmeans update");
  }
  return commit_staged(c);
}

qwm_status qwm_import_calibration(qwm_cache* c, const void* C, const float* S_G, const float* U_r) {
  qwm_status st;
  if ((st = check_cache(c)) != QWM_OK) return st;
  if ((st = check_ptr(C, "C")) != QWM_OK) return st;
  if (S_G || c->obj == qwm::kObjQsac)
    if ((st = check_ptr(S_G, "S_G")) != QWM_OK) return st;
  if (U_r || c->r > 0)
    if ((st = check_ptr(U_r, "U_r")) != QWM_OK) return st;
  if (!epoch_room(c)) return fail(QWM_ERR_CAPACITY, "max_epochs reached");
  if ((st = need_device(c)) != QWM_OK) return st;
  DeviceGuard g(c->device);
  const int stg = c->staged();
  hipError_t e;
  if ((e = c->join_side()) != hipSuccess) return fail_hip(e, "join eigensolve");
  if ((e = hipMemcpyAsync(c->slotC(stg), C, (size_t)c->H * c->m * c->D * c->esz, hipMemcpyDeviceToDevice,
                          c->stream)) != hipSuccess)
    return fail_hip(e, "import C");
  if (S_G) {
    if ((e = hipMemcpyAsync(c->slotS(stg), S_G, (size_t)c->H * c->nG * 4, hipMemcpyDeviceToDevice, c->stream)) !=
        hipSuccess)
      return fail_hip(e, "import S");
  } else {
    e = c->run(QWM_K_OTHER, [&] { return qwm::launch_fill(c->slotS(stg), (int64_t)c->H * c->nG, 0.0f, c->stream); });
    if (e != hipSuccess) return fail_hip(e, "zero sensitivity");
  }
  if (c->r > 0 && (e = hipMemcpyAsync(c->slotU(stg), U_r, (size_t)c->H * c->D * c->r * 4, hipMemcpyDeviceToDevice,
                                      c->stream)) != hipSuccess)
    return fail_hip(e, "import U");
  return commit_staged(c);
}

qwm_status qwm_export_calibration(const qwm_cache* cc, int32_t epoch, void* C, float* S_G, float* U_r) {
  qwm_status st;
  if ((st = check_cache(cc)) != QWM_OK) return st;
  qwm_cache* c = const_cast<qwm_cache*>(cc);
  if (epoch < -1 || epoch >= (int)c->epoch_start.size()) return fail(QWM_ERR_INVALID_ARG, "no such epoch");
  const int slot = epoch < 0 ? c->staged() : epoch;
  if ((st = need_device(c)) != QWM_OK) return st;
  DeviceGuard g(c->device);
  hipError_t e;
  if ((e = c->join_side()) != hipSuccess) return fail_hip(e, "join eigensolve");
  if (C && (e = hipMemcpyAsync(C, c->slotC(slot), (size_t)c->H * c->m * c->D * c->esz, hipMemcpyDeviceToDevice,
                               c->stream)) != hipSuccess)
    return fail_hip(e, "export C");
  if (S_G && (e = hipMemcpyAsync(S_G, c->slotS(slot), (size_t)c->H * c->nG * 4, hipMemcpyDeviceToDevice,
                                 c->stream)) != hipSuccess)
    return fail_hip(e, "export S");
  if (U_r && c->r > 0 && (e = hipMemcpyAsync(U_r, c->slotU(slot), (size_t)c->H * c->D * c->r * 4, hipMemcpyDeviceToDevice,
                                 c->stream)) != hipSuccess)
    return fail_hip(e, "export U");
  return QWM_OK;
}

qwm_status qwm_quantize_append(qwm_cache* c, const void* k, const void* v, int64_t n_tokens) {
  qwm_status st;
  if ((st = check_cache(c)) != QWM_OK) return st;
  if (n_tokens != 0) {  // with no tokens nothing is read: k and v may be NULL
    if ((st = check_ptr(k, "k")) != QWM_OK) return st;
    if ((st = check_ptr(v, "v")) != QWM_OK) return st;
  }
  if (n_tokens < 0) return fail(QWM_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (c->epoch_start.empty()) return fail(QWM_ERR_STATE, "quantize_append before a committed epoch");
  if (c->length + n_tokens > c->desc.capacity_tokens) return fail(QWM_ERR_CAPACITY, "capacity exceeded");
  if (n_tokens == 0) return QWM_OK;
  if ((st = need_device(c)) != QWM_OK) return st;
  DeviceGuard g(c->device);
  const int slot = (int)c->epoch_start.size() - 1;
  qwm::QuantArgs a{};
  a.k = k;
  a.v = v;
  a.n = n_tokens;
  a.C32 = c->C32();
  a.S = c->slotS(slot);
  a.U64 = c->U64();
  a.cache = c->view;
  a.pos0 = c->length;
  a.H = c->H;
  a.m = c->m;
  a.r = c->r;
  a.obj = c->obj;
  // (no split here: the finishing pass would serialize the quantization and
  // PSAC phase, which the whole kernel overlaps with other blocks' scans)
  hipError_t e = c->run(QWM_K_QUANTIZE, [&] { return qwm::launch_quantize(c->D, c->dtype, a, c->stream); });
  if (e == hipSuccess) c->count_full_pass(QWM_K_QUANTIZE, n_tokens);
  if (e != hipSuccess) return fail_hip(e, "quantize");
  c->length += n_tokens;
  return QWM_OK;
}

qwm_status qwm_attend(qwm_cache* c, const void* q, int64_t n_q, const void* k_self, const void* v_self,
                      int64_t n_self, int32_t mask, float softmax_scale, float* out) {
  qwm_status st = check_attend(c, q, n_q, k_self, v_self, n_self, mask, softmax_scale, out, true);
  if (st != QWM_OK) return st;
  DeviceGuard g(c->device);
  return attend_impl(c, q, n_q, k_self, v_self, n_self, mask, softmax_scale, out, arena_work(c));
}

qwm_status qwm_attend_noalloc(qwm_cache* c, const void* q, int64_t n_q, const void* k_self, const void* v_self,
                              int64_t n_self, int32_t mask, float softmax_scale, float* out) {
  qwm_status st = check_attend(c, q, n_q, k_self, v_self, n_self, mask, softmax_scale, out, false);
  if (st != QWM_OK) return st;
  DeviceGuard g(c->device);
  uint8_t* base = nullptr;
  if ((st = static_scratch(c->device, &base)) != QWM_OK) return st;
  // carve the call's tables out of the static scratch; the partials take
  // what is left (splits are cut to fit, down to none)
  const size_t E = c->epoch_start.size(), H = (size_t)c->H;
  const bool decode = use_decode(c, mask, n_q);
  const size_t nqp = (size_t)((n_q + qwm::kDecodeQ - 1) / qwm::kDecodeQ * qwm::kDecodeQ);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t oU = take(H * E * (size_t)n_q * qwm::kRankPad * 4);
  const size_t oC = decode ? take(H * E * (size_t)c->m * nqp * 4) : off;
  // the fp16 centroid copy of the bf16 head_dim-128 prefill path, where it
  // fits (without it the kernel converts the bf16 rows of every tile)
  const size_t c16_bytes = H * E * (size_t)c->m * c->D * 2;
  const bool c16 = !decode && c->dtype == QWM_BF16 && c->D == 128 && align_up(off + c16_bytes) + 2 * kAlign <= kScratchBytes;
  const size_t oC16 = c16 ? take(c16_bytes) : 0;
  if (off + 2 * kAlign > kScratchBytes)
    return fail(QWM_ERR_CAPACITY, "qwm_attend_noalloc: n_q = " + std::to_string(n_q) + " needs " + std::to_string(off) +
                                      " bytes of tables, beyond the " + std::to_string(kScratchBytes >> 20) +
                                      " MiB static scratch");
  const size_t rows = (kScratchBytes - off - 2 * kAlign) / ((size_t)c->D * 4 + 8);
  const size_t oO = take(rows * c->D * 4), oML = take(rows * 8);
  AttnWork w{reinterpret_cast<float*>(base + oU), reinterpret_cast<float*>(base + oC),
             reinterpret_cast<float*>(base + oO), reinterpret_cast<float*>(base + oML), (int64_t)rows,
             c16 ? static_cast<void*>(base + oC16) : nullptr};
  c->no_events = true;  // hipEventCreate is not called on this path
  st = attend_impl(c, q, n_q, k_self, v_self, n_self, mask, softmax_scale, out, w);
  c->no_events = false;
  return st;
}

qwm_status qwm_attend_logits(qwm_cache* c, const void* q, int64_t n_q, int32_t head, float softmax_scale,
                             float* logits) {
  qwm_status st;
  if ((st = check_cache(c)) != QWM_OK) return st;
  if ((st = check_ptr(q, "q")) != QWM_OK) return st;
  if ((st = check_ptr(logits, "logits")) != QWM_OK) return st;
  if (n_q < 1) return fail(QWM_ERR_INVALID_ARG, "n_q must be >= 1");
  if (n_q > c->desc.max_query_tokens) return fail(QWM_ERR_CAPACITY, "n_q exceeds max_query_tokens");
  if (head < 0 || head >= c->H) return fail(QWM_ERR_INVALID_ARG, "head out of range");
  if (!std::isfinite(softmax_scale)) return fail(QWM_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (c->epoch_start.empty() || c->length == 0) return fail(QWM_ERR_STATE, "empty cache");
  if ((st = need_device(c)) != QWM_OK) return st;
  DeviceGuard g(c->device);
  qwm::AttnPlan p;
  make_plan(c, 0, false, p);
  const int T = p.tile_prefix[p.n_seg];
  const int E = (int)c->epoch_start.size();
  qwm::AttnArgs a = base_args(c, arena_work(c));
  a.q = q;
  a.qU = c->qU();
  a.nq = n_q;
  a.scale = softmax_scale;
  a.n_epoch_slots = E;
  a.qpb = queries_per_block(n_q);
  a.logits = logits;
  a.logit_head = head;
  a.logit_len = c->length;
  a.splits = T < 64 ? T : 64;
  hipError_t e = hipSuccess;
  if (c->r > 0) {  // the kernels read no qU at rank 0
    e = c->run(QWM_K_QU, [&] {
      return qwm::launch_qu(c->D, c->dtype, q, n_q, c->H, c->r, c->slotU(0), (int64_t)c->H * c->D * c->r, E, c->qU(),
                            c->stream);
    });
    if (e != hipSuccess) return fail_hip(e, "qU");
  }
  e = c->run(QWM_K_ATTEND, [&] { return qwm::launch_attend_logits(c->D, c->dtype, a, p, c->stream); });
  if (e != hipSuccess) return fail_hip(e, "attend_logits");
  return QWM_OK;
}

qwm_status qwm_attend_top1(qwm_cache* c, const void* q, int64_t n_q, const void* k_ref, int64_t n_ref,
                           int32_t* top1) {
  qwm_status st;
  if ((st = check_cache(c)) != QWM_OK) return st;
  if ((st = check_ptr(q, "q")) != QWM_OK) return st;
  if ((st = check_ptr(top1, "top1")) != QWM_OK) return st;
  if (n_q < 1) return fail(QWM_ERR_INVALID_ARG, "n_q must be >= 1");
  if (n_q > c->desc.max_query_tokens) return fail(QWM_ERR_CAPACITY, "n_q exceeds max_query_tokens");
  const bool ref = (k_ref != nullptr);
  if (ref) {
    if ((st = check_ptr(k_ref, "k_ref")) != QWM_OK) return st;
    if (n_ref < 1) return fail(QWM_ERR_INVALID_ARG, "n_ref must be >= 1 with k_ref");
    if (n_ref > ((int64_t)1 << 22)) return fail(QWM_ERR_CAPACITY, "n_ref beyond 2^22");
  } else {
    if (n_ref != 0) return fail(QWM_ERR_INVALID_ARG, "n_ref must be 0 without k_ref");
    if (c->epoch_start.empty() || c->length == 0) return fail(QWM_ERR_STATE, "empty cache");
  }
  if ((st = need_device(c)) != QWM_OK) return st;
  DeviceGuard g(c->device);
  qwm::AttnPlan p;
  if (ref) {  // one segment: the full-precision Keys
    std::memset(&p, 0, sizeof(p));
    p.n_seg = 1;
    p.seg_start[0] = 0;
    p.seg_len[0] = (int32_t)n_ref;
    p.seg_epoch[0] = -1;
    p.tile_prefix[1] = (int32_t)((n_ref + qwm::kTileKV - 1) / qwm::kTileKV);
  } else {
    make_plan(c, 0, false, p);
  }
  const int T = p.tile_prefix[p.n_seg];
  const int E = (int)c->epoch_start.size();
  qwm::AttnArgs a = base_args(c, arena_work(c));
  a.q = q;
  a.qU = c->qU();
  a.kself = ref ? k_ref : nullptr;
  a.nq = n_q;
  a.nself = ref ? n_ref : 0;
  a.scale = 1.0f;
  a.scale_log2 = 1.4426950408889634f;
  a.n_epoch_slots = E;
  a.qpb = queries_per_block(n_q);
  a.top1 = top1;
  a.splits = choose_splits(c, n_q, T, c->L.part_rows);
  hipError_t e = hipSuccess;
  if (!ref && c->r > 0) {
    e = c->run(QWM_K_QU, [&] {
      return qwm::launch_qu(c->D, c->dtype, q, n_q, c->H, c->r, c->slotU(0), (int64_t)c->H * c->D * c->r, E, c->qU(),
                            c->stream);
    });
    if (e != hipSuccess) return fail_hip(e, "qU");
  }
  e = c->run(QWM_K_ATTEND, [&] { return qwm::launch_attend_top1(c->D, c->dtype, a, p, c->stream); });
  if (e != hipSuccess) return fail_hip(e, "attend_top1");
  if (a.splits > 1) {
    e = c->run(QWM_K_MERGE, [&] { return qwm::launch_top1_merge(a, c->stream); });
    if (e != hipSuccess) return fail_hip(e, "top1 merge");
  }
  return QWM_OK;
}

qwm_status qwm_length(const qwm_cache* c, int64_t* n_tokens) {
  if (!c || !n_tokens) return fail(QWM_ERR_INVALID_ARG, "NULL argument");
  *n_tokens = c->length;
  return QWM_OK;
}

qwm_status qwm_epochs(const qwm_cache* c, int32_t* n_epochs) {
  if (!c || !n_epochs) return fail(QWM_ERR_INVALID_ARG, "NULL argument");
  *n_epochs = (int32_t)c->epoch_start.size();
  return QWM_OK;
}

qwm_status qwm_truncate(qwm_cache* c, int64_t n_tokens) {
  if (!c) return fail(QWM_ERR_INVALID_ARG, "cache is NULL");
  if (n_tokens < 0 || n_tokens > c->length) return fail(QWM_ERR_INVALID_ARG, "n_tokens must be in [0, length]");
  const size_t before = c->epoch_start.size();
  c->length = n_tokens;
  while (c->epoch_start.size() > 1 && c->epoch_start.back() > n_tokens) c->epoch_start.pop_back();
  if (c->epoch_start.size() != before && !c->epoch_start.empty()) {
    qwm_status st;
    if ((st = need_device(c)) != QWM_OK) return st;
    DeviceGuard g(c->device);
    const int slot = (int)c->epoch_start.size() - 1;
    hipError_t e = c->run(QWM_K_OTHER, [&] {
      return qwm::launch_shadow(c->D, c->dtype, c->slotC(slot), c->slotU(slot), c->H, c->m, c->r, c->C32(),
                                c->U64(), c->stream);
    });
    if (e != hipSuccess) return fail_hip(e, "shadow");
  }
  return QWM_OK;
}

qwm_status qwm_export_bytes(const qwm_cache* c, int64_t t0, int64_t t1, size_t* bytes) {
  if (!c || !bytes) return fail(QWM_ERR_INVALID_ARG, "NULL argument");
  if (t0 < 0 || t1 < t0 || t1 > c->length) return fail(QWM_ERR_INVALID_ARG, "need 0 <= t0 <= t1 <= length");
  *bytes = (size_t)c->H * (size_t)(t1 - t0) * (size_t)(c->D / 2 + 8 * c->nG + 1 + 2 * c->r + 2);
  return QWM_OK;
}

qwm_status qwm_export(const qwm_cache* cc, int64_t t0, int64_t t1, void* dev_buf) {
  if (!cc) return fail(QWM_ERR_INVALID_ARG, "cache is NULL");
  if (!dev_buf) return fail(QWM_ERR_INVALID_ARG, "dev_buf is NULL");
  if (t0 < 0 || t1 < t0 || t1 > cc->length) return fail(QWM_ERR_INVALID_ARG, "need 0 <= t0 <= t1 <= length");
  qwm_cache* c = const_cast<qwm_cache*>(cc);
  qwm_status st;
  if ((st = need_device(c)) != QWM_OK) return st;
  DeviceGuard g(c->device);
  qwm::ExportArgs a{};
  a.cache = c->view;
  a.t0 = t0;
  a.n = t1 - t0;
  a.n_epochs = (int)c->epoch_start.size();
  for (int i = 0; i < a.n_epochs; ++i) a.epoch_start[i] = (int32_t)c->epoch_start[i];
  a.H = c->H;
  a.D = c->D;
  a.nG = c->nG;
  a.r = c->r;
  a.out = reinterpret_cast<uint8_t*>(dev_buf);
  hipError_t e = c->run(QWM_K_OTHER, [&] { return qwm::launch_export(a, c->stream); });
  if (e != hipSuccess) return fail_hip(e, "export");
  return QWM_OK;
}

qwm_status qwm_profile_enable(qwm_cache* c, int32_t enable) {
  if (!c) return fail(QWM_ERR_INVALID_ARG, "cache is NULL");
  for (auto& rec : c->pending) {
    (void)hipEventDestroy(rec.a);
    (void)hipEventDestroy(rec.b);
  }
  c->pending.clear();
  for (int i = 0; i < QWM_K_COUNT; ++i) {
    c->prof_ms[i] = 0.0;
    c->prof_n[i] = 0;
    c->work_host[i] = 0.0;
  }
  c->work_clear = true;
  c->profile = enable != 0;
  return QWM_OK;
}

qwm_status qwm_profile_read(qwm_cache* c, int32_t kid, double* total_ms, int64_t* launches) {
  if (!c || !total_ms || !launches) return fail(QWM_ERR_INVALID_ARG, "NULL argument");
  if (kid < 0 || kid >= QWM_K_COUNT) return fail(QWM_ERR_INVALID_ARG, "bad kernel id");
  qwm_status st;
  if (!c->pending.empty() && (st = need_device(c)) != QWM_OK) return st;
  DeviceGuard g(c->device);
  for (auto& rec : c->pending) {
    hipError_t e = hipEventSynchronize(rec.b);
    if (e != hipSuccess) return fail_hip(e, "profile sync");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, rec.a, rec.b);
    if (e != hipSuccess) return fail_hip(e, "profile elapsed");
    c->prof_ms[rec.kid] += ms;
    c->prof_n[rec.kid] += 1;
    (void)hipEventDestroy(rec.a);
    (void)hipEventDestroy(rec.b);
  }
  c->pending.clear();
  *total_ms = c->prof_ms[kid];
  *launches = c->prof_n[kid];
  return QWM_OK;
}

qwm_status qwm_profile_work(qwm_cache* c, int32_t kid, double* evaluations) {
  if (!c || !evaluations) return fail(QWM_ERR_INVALID_ARG, "NULL argument");
  if (kid < 0 || kid >= QWM_K_COUNT) return fail(QWM_ERR_INVALID_ARG, "bad kernel id");
  unsigned long long dev_count = 0;
  if (!c->work_clear) {  // a pruned launch wrote the counters since profiling was enabled
    qwm_status st;
    if ((st = need_device(c)) != QWM_OK) return st;
    DeviceGuard g(c->device);
    hipError_t e = hipMemcpyAsync(&dev_count, c->work() + kid, sizeof(dev_count), hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return fail_hip(e, "profile work read");
  }
  *evaluations = c->work_host[kid] + (double)dev_count;
  return QWM_OK;
}

}  // extern "C"
