// C-ABI entry points: argument checks, kernel selection, launches on the caller's stream,
// optional contract validation (PAGEDKV_VALIDATE=1) and kernel timing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "kernels.h"
#include "pagedkv.h"
#include "schedule.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return PKV_OK;
}

int env_int(const char* name, int dflt) {
  const char* e = std::getenv(name);
  if (!e || !*e) return dflt;
  return std::atoi(e);
}

int g_validate = -1;   // -1: not decided yet, then 0 / 1

bool validate_mode() {
  if (g_validate < 0) g_validate = env_int("PAGEDKV_VALIDATE", 0) != 0 ? 1 : 0;
  return g_validate == 1;
}

int elem_bytes(int dt) {
  if (dt == PKV_F32) return 4;
  if (dt == PKV_F16 || dt == PKV_BF16) return 2;
  return 0;
}

int launch_error(hipError_t e, const char* what) {
  return fail(PKV_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
}

// ---- kernel timing --------------------------------------------------------------------
struct TimingRec {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_tmu;
bool g_timing = false;
int g_timing_every = 1;                       // time every k-th launch of each kernel
std::vector<std::pair<const char*, int64_t>> g_seen;   // launches per kernel name
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_spare;

hipEvent_t take_event() {
  if (!g_spare.empty()) {
    hipEvent_t e = g_spare.back();
    g_spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace pkv {
LaunchEvents& launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}
}  // namespace pkv

namespace {

template <class F>
hipError_t timed(const char* name, hipStream_t st, F&& launch) {
  std::unique_lock<std::mutex> lk(g_tmu);
  if (!g_timing) {
    lk.unlock();
    return launch();
  }
  int64_t* seen = nullptr;
  for (auto& x : g_seen)
    if (x.first == name) seen = &x.second;
  if (!seen) {
    g_seen.push_back({name, 0});
    seen = &g_seen.back().second;
  }
  if ((*seen)++ % g_timing_every != 0) {
    lk.unlock();
    return launch();
  }
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return hipErrorOutOfMemory;
  // the first kernel the call launches stamps a and b with its own start and end
  pkv::LaunchEvents& ev = pkv::launch_events();
  ev = pkv::LaunchEvents{a, b, false};
  hipError_t e = launch();
  const bool stamped = ev.used;
  ev = pkv::LaunchEvents{};
  hipError_t e2 = hipSuccess;
  if (!stamped) {   // nothing was launched (an empty call): a zero-length interval
    e2 = hipEventRecord(a, st);
    if (e2 == hipSuccess) e2 = hipEventRecord(b, st);
  }
  g_recs.push_back({name, a, b});
  return e != hipSuccess ? e : e2;
}

// ---- host copies for PAGEDKV_VALIDATE ------------------------------------------------
bool copy_ints(std::vector<int32_t>& dst, const int32_t* src, size_t n, hipStream_t st) {
  dst.resize(n);
  if (n == 0) return true;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
      hipSuccess)
    return false;
  return hipStreamSynchronize(st) == hipSuccess;
}

// Upper bound of the automatic worker count per compute unit (two resident wavefronts per SIMD,
// four SIMDs); the automatic workspace size assumes it, the kernels' actual residency (one
// wavefront per SIMD for the matrix-core kernel) is never above it.
constexpr int kWorkersPerCU = 8;

int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev] = v;
  return v;
}

// Resident wavefronts per CU of a decode kernel configuration (the occupancy query costs
// tens of microseconds of host time, so each configuration is asked once per device).
int resident_waves_cached(bool mfma, int kv_dtype, int head_dim, int block_size, int G,
                          int waves, int num_seqs) {
  struct Key {
    int dev, mfma, dt, d, b, g, w, s;
    bool operator==(const Key& o) const {
      return dev == o.dev && mfma == o.mfma && dt == o.dt && d == o.d && b == o.b && g == o.g &&
             w == o.w && s == o.s;
    }
  };
  static std::mutex mu;
  static std::vector<std::pair<Key, int>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const Key k{dev, mfma ? 1 : 0, kv_dtype, head_dim, block_size, G, waves, num_seqs};
  {
    std::lock_guard<std::mutex> lk(mu);
    for (auto& e : cache)
      if (e.first == k) return e.second;
  }
  const int v = mfma ? pkv::decode_mfma_resident_waves(kv_dtype, head_dim, block_size, G, waves,
                                                       num_seqs)
                     : pkv::decode_valu_resident_waves(kv_dtype, head_dim, block_size, G, waves,
                                                       num_seqs);
  std::lock_guard<std::mutex> lk(mu);
  if (cache.size() < 4096) cache.push_back({k, v});
  return v;
}

int choose_workers(int num_workers) {
  return num_workers > 0 ? num_workers : pkv_decode_auto_workers();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Schedule weight of a segment start relative to a step's 4. With streaming (non-temporal)
// key/value loads a piece start costs about a quarter of a step on gfx950: per-wavefront
// timestamps on the GQA batch put a step at about 2 us and a piece start at no measurable
// extra time, and of the weights 4, 2, 1 and 0, weight 1 gave the shortest decode at both
// block sizes. PAGEDKV_PIECE_WEIGHT overrides it for measurements (read once per process).
int piece_weight() {
  static const int v = [] {
    const int x = env_int("PAGEDKV_PIECE_WEIGHT", 1);
    return x < 0 ? 0 : (x > 64 ? 64 : x);
  }();
  return v;
}

struct WsLayout {
  size_t prefix, wprefix, m, l, acc, total;
};

// Two partial slots per worker, and the two per-sequence prefixes the merge reads.
WsLayout ws_layout(int num_seqs, int G, int head_dim, int n) {
  const size_t slots = 2 * (size_t)n;
  WsLayout L;
  L.prefix = 0;
  L.wprefix = align256(((size_t)num_seqs + 1) * sizeof(int64_t));
  L.m = L.wprefix + align256(((size_t)num_seqs + 1) * sizeof(int64_t));
  L.l = L.m + align256(slots * G * sizeof(float));
  L.acc = L.l + align256(slots * G * sizeof(float));
  L.total = L.acc + align256(slots * G * head_dim * sizeof(float));
  return L;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_err.c_str(); }

const char* pkv_version(void) { return "pagedkv-gfx950 0.1"; }

int pkv_decode_auto_workers(void) {
  const int cus = cu_count();
  return cus > 0 ? cus * kWorkersPerCU : 256 * kWorkersPerCU;
}

size_t pkv_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int num_workers) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_q_heads % num_kv_heads != 0 || num_workers < 0)
    return 0;
  return ws_layout(num_seqs, num_q_heads / num_kv_heads, head_dim, choose_workers(num_workers))
      .total;
}

}  // extern "C"

namespace {

// Shared-prefix mode of the decode: the decode writes normalised fp32 rows to `out` and their
// log-sum-exp to lse; the merge folds every segment with the prefix states and writes the
// results to final_out. The caller has validated the device contents.
struct PrefixFold {
  float* lse;
  void* final_out;
  int final_f32;
  const float* m;
  const float* l;
  const float* acc;
  int groups;
};

// More query heads per KV head than one decode segment takes (16 on the matrix cores; 1, 2, 4
// or 8 for fp32 caches, on the VALU kernel) run as kv_split schedule heads of G / kv_split
// query heads each over the same pool KV head: the smallest such split (1 when G fits).
int kv_split_for(int G, bool wide) {
  for (int k = 1; k < G; ++k) {
    if (G % k != 0) continue;
    const int gv = G / k;
    if (wide ? gv <= 16 : (gv == 1 || gv == 2 || gv == 4 || gv == 8)) return k;
  }
  return G > 0 ? G : 1;   // one query head per schedule head
}

// Decode (paged_attn_decode), optionally with each sequence's newest token taken from k_new /
// v_new and stored into its slot by the same kernel (paged_attn_decode_append).
int decode_impl(const char* fn, void* out, int out_dtype, const void* q, const void* k_pool,
                const void* v_pool, int kv_dtype, const void* k_new, const void* v_new,
                const int32_t* block_tables, int max_blocks_per_seq,
                const int32_t* context_lens, int max_context_len, int num_seqs,
                int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                float scale, int num_workers, void* workspace, size_t workspace_bytes,
                void* stream, const PrefixFold* pf = nullptr) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || max_context_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: non-positive size", fn);
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (elem_bytes(kv_dtype) == 0)
    return fail(PKV_ERR_UNSUPPORTED, "%s: kv_dtype %d", fn, kv_dtype);
  if (!(out_dtype == PKV_F32 || out_dtype == kv_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "%s: out_dtype %d with kv_dtype %d", fn,
                out_dtype, kv_dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, head_dim);
  if (block_size != 16 && block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "%s: block_size %d (16 or 32)", fn, block_size);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: %d query heads not a multiple of %d KV heads", fn,
                num_q_heads, num_kv_heads);
  const bool wide = kv_dtype != PKV_F32;
  // the schedule's KV heads and query heads per KV head (kv_split per pool KV head)
  const int kv_split = kv_split_for(num_q_heads / num_kv_heads, wide);
  const int pool_kv_heads = num_kv_heads;
  num_kv_heads *= kv_split;
  const int G = num_q_heads / num_kv_heads;
  bool use_mfma;
  // the suffix decode of a shared-prefix call takes the matrix-core kernel at G = 1 too: only
  // it writes the rows' log-sum-exp that the prefix fold needs
  if (wide && ((G >= 2 && G <= 16) || (G == 1 && pf))) {
    use_mfma = true;
  } else if (G == 1 || (!wide && (G == 2 || G == 4 || G == 8))) {
    use_mfma = false;
  } else {
    return fail(PKV_ERR_UNSUPPORTED, "%s: %d query heads per KV head", fn, G);
  }
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_ERR_INVALID_ARG,
                "%s: max_context_len %d exceeds table capacity %d x %d", fn,
                max_context_len, max_blocks_per_seq, block_size);
  if (num_workers < 0 || num_workers > (1 << 20))
    return fail(PKV_ERR_INVALID_ARG, "%s: num_workers %d", fn, num_workers);
  if (num_seqs > pkv::kMaxSeqsPerCall) {
    // A launch's schedule keeps its sequences' prefixes in LDS: more sequences run as
    // consecutive launches of at most kMaxSeqsPerCall sequences on the caller's stream, each
    // reusing the workspace (sized for all of them, so large enough for any part). Sequences
    // are independent, so the results are those of one launch over all of them.
    if (pf)
      return fail(PKV_ERR_UNSUPPORTED, "%s: %d sequences (at most %d per call)", fn, num_seqs,
                  pkv::kMaxSeqsPerCall);
    const size_t qb = (size_t)num_q_heads * head_dim * elem_bytes(kv_dtype);
    const size_t ob = (size_t)num_q_heads * head_dim * elem_bytes(out_dtype);
    const size_t nb = (size_t)pool_kv_heads * head_dim * elem_bytes(kv_dtype);
    for (int s0 = 0; s0 < num_seqs; s0 += pkv::kMaxSeqsPerCall) {
      const int ns = std::min(pkv::kMaxSeqsPerCall, num_seqs - s0);
      const int rc = decode_impl(
          fn, reinterpret_cast<char*>(out) + s0 * ob, out_dtype,
          reinterpret_cast<const char*>(q) + s0 * qb, k_pool, v_pool, kv_dtype,
          k_new ? reinterpret_cast<const char*>(k_new) + s0 * nb : nullptr,
          v_new ? reinterpret_cast<const char*>(v_new) + s0 * nb : nullptr,
          block_tables + (size_t)s0 * max_blocks_per_seq, max_blocks_per_seq,
          context_lens + s0, max_context_len, ns, num_q_heads, pool_kv_heads, head_dim,
          block_size, num_blocks, scale, num_workers, workspace, workspace_bytes, stream);
      if (rc != PKV_OK) return rc;
    }
    return ok();
  }
  static const int waves_env = env_int("PAGEDKV_DECODE_WAVES", 4);
  const int waves = (waves_env == 1 || waves_env == 2 || waves_env == 4) ? waves_env : 4;
  int n = num_workers;
  if (n == 0) {
    // every worker resident at once: the resident wavefronts per CU of the chosen kernel,
    // capped by the per-CU count the automatic workspace size assumes
    int per_cu = resident_waves_cached(use_mfma, kv_dtype, head_dim, block_size, G, waves,
                                       num_seqs);
    if (per_cu <= 0 || per_cu > kWorkersPerCU) per_cu = kWorkersPerCU;
    const int cus = cu_count();
    n = (cus > 0 ? cus : 256) * per_cu;
    // no more workers than the line can have steps: a worker past them would only pay the
    // schedule prologue, and every extra range boundary is one more partial to merge
    const int64_t max_steps = (int64_t)num_kv_heads * num_seqs *
                              ((max_context_len + pkv::kStepTokens - 1) / pkv::kStepTokens);
    if (max_steps < n) n = (int)std::max<int64_t>(max_steps, 1);
  }
  const int pw = piece_weight();
  {
    // the weighted step line must fit the 64-bit worker arithmetic: N_w * n < 2^62
    const double weight_max = (double)num_kv_heads * num_seqs *
                              (4.0 * ((double)max_context_len / 32.0 + 1.0) + pw);
    if (weight_max * (double)n >= 4.0e18)
      return fail(PKV_ERR_UNSUPPORTED, "%s: problem too large for one call", fn);
  }
  const WsLayout wl = ws_layout(num_seqs, G, head_dim, n);
  if (!workspace || workspace_bytes < wl.total)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn,
                workspace_bytes, wl.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(PKV_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", fn);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  if (!pf && validate_mode()) {
    std::vector<int32_t> lens, tabs;
    if (!copy_ints(lens, context_lens, num_seqs, st) ||
        !copy_ints(tabs, block_tables, (size_t)num_seqs * max_blocks_per_seq, st))
      return fail(PKV_ERR_LAUNCH, "%s: validation copy failed", fn);
    for (int s = 0; s < num_seqs; ++s) {
      if (lens[s] < 0 || lens[s] > max_context_len)
        return fail(PKV_ERR_VALIDATION, "context_lens[%d] = %d outside [0, %d]", s, lens[s],
                    max_context_len);
      const int nb = (lens[s] + block_size - 1) / block_size;
      for (int j = 0; j < nb; ++j) {
        const int b = tabs[(size_t)s * max_blocks_per_seq + j];
        if (b < 0 || b >= num_blocks)
          return fail(PKV_ERR_VALIDATION, "block_tables[%d][%d] = %d outside [0, %d)", s, j, b,
                      num_blocks);
      }
    }
  }

  pkv::DecodeParams p{};
  p.out = out;
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_pool_w = k_new ? const_cast<void*>(k_pool) : nullptr;
  p.v_pool_w = k_new ? const_cast<void*>(v_pool) : nullptr;
  p.tables = block_tables;
  p.lens = context_lens;
  p.out_f32 = out_dtype == PKV_F32 ? 1 : 0;
  p.max_blocks = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.kv_split = kv_split;
  p.pool_kv_heads = pool_kv_heads;
  p.num_blocks = num_blocks;
  p.block_size = block_size;
  p.num_workers = n;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)head_dim);
  p.scale_log2 = sc * 1.4426950408889634f;
  p.piece_weight = pw;
  // streaming key/value loads for a decode that reads its blocks once; the suffix decode of the
  // shared-prefix call (short segments right after the prefix pass) runs faster with plain ones
  p.stream_loads = (pf && use_mfma && waves == 4) ? 0 : 1;
  p.ring_cap = pkv::ring_capacity(num_seqs, G, head_dim, waves);
  char* ws = reinterpret_cast<char*>(workspace);
  p.wprefix = reinterpret_cast<int64_t*>(ws + wl.wprefix);
  p.ws_acc = reinterpret_cast<float*>(ws + wl.acc);
  p.ws_m = reinterpret_cast<float*>(ws + wl.m);
  p.ws_l = reinterpret_cast<float*>(ws + wl.l);
  p.prefix = reinterpret_cast<int64_t*>(ws + wl.prefix);
  p.final_out = out;
  p.final_f32 = p.out_f32;
  if (pf) {
    p.lse = pf->lse;
    p.final_out = pf->final_out;
    p.final_f32 = pf->final_f32;
    p.pst_m = pf->m;
    p.pst_l = pf->l;
    p.pst_acc = pf->acc;
    p.pst_groups = pf->groups;
  }

  hipError_t e;
  if (use_mfma) {
    e = timed("decode_partial_mfma", st, [&] {
      return pkv::launch_decode_mfma(p, kv_dtype, head_dim, block_size, waves, st);
    });
  } else {
    e = timed("decode_partial_valu", st, [&] {
      return pkv::launch_decode_valu(p, kv_dtype, head_dim, block_size, G, waves, st);
    });
  }
  if (e != hipSuccess)
    return fail(PKV_ERR_LAUNCH, "%s: decode kernel: %s", fn, hipGetErrorString(e));
  e = timed("splitk_reduce", st,
            [&] { return pkv::launch_splitk_reduce(p, kv_dtype, head_dim, st); });
  if (e != hipSuccess)
    return fail(PKV_ERR_LAUNCH, "%s: merge kernel: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int paged_attn_decode(void* out, int out_dtype, const void* q, const void* k_pool,
                      const void* v_pool, int kv_dtype, const int32_t* block_tables,
                      int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, float scale, int num_workers,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl("paged_attn_decode", out, out_dtype, q, k_pool, v_pool, kv_dtype, nullptr,
                     nullptr, block_tables, max_blocks_per_seq, context_lens, max_context_len,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     num_workers, workspace, workspace_bytes, stream);
}

}  // extern "C"

// Scratch of paged_attn_decode_noalloc: a static device array (one copy per GPU, zero at
// load, held until the process ends). Host code never uses the array's name as an address:
// its device address is looked up once per device, with that device current, and kept.
static __device__ __align__(256) unsigned char scratch[PKV_DECODE_STATIC_SCRATCH];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, or nullptr (error message set).
void* scratch_address(const char* fn) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fail(PKV_ERR_LAUNCH, "%s: no usable current device", fn);
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(PKV_ERR_LAUNCH, "%s: hipGetSymbolAddress of the static scratch: %s", fn,
           hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int paged_attn_decode_noalloc(void* out, int out_dtype, const void* q, const void* k_pool,
                              const void* v_pool, int kv_dtype, const int32_t* block_tables,
                              int max_blocks_per_seq, const int32_t* context_lens,
                              int max_context_len, int num_seqs, int num_q_heads,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                              float scale, int num_workers, void* stream) {
  const char* fn = "paged_attn_decode_noalloc";
  if (num_seqs == 0) return ok();
  if (num_seqs > 0 && num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0 &&
      head_dim > 0 && num_workers >= 0) {
    const size_t need = pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                  num_workers);
    if (need > PKV_DECODE_STATIC_SCRATCH)
      return fail(PKV_ERR_WORKSPACE_TOO_SMALL,
                  "%s: the call needs %zu bytes of scratch, the static array holds %zu", fn,
                  need, (size_t)PKV_DECODE_STATIC_SCRATCH);
  }
  void* ws = scratch_address(fn);
  if (!ws) return PKV_ERR_LAUNCH;
  return decode_impl(fn, out, out_dtype, q, k_pool, v_pool, kv_dtype, nullptr, nullptr,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     num_workers, ws, PKV_DECODE_STATIC_SCRATCH, stream);
}

int paged_attn_decode_append(void* out, int out_dtype, const void* q, void* k_pool, void* v_pool,
                             int kv_dtype, const void* k_new, const void* v_new,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len, int num_seqs,
                             int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                             int num_blocks, float scale, int num_workers, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new))
    return fail(PKV_ERR_INVALID_ARG, "paged_attn_decode_append: null pointer");
  return decode_impl("paged_attn_decode_append", out, out_dtype, q, k_pool, v_pool, kv_dtype,
                     k_new, v_new, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, scale, num_workers, workspace, workspace_bytes, stream);
}

int kv_cache_append(void* k_pool, void* v_pool, int kv_dtype, const void* k_new,
                    const void* v_new, const int32_t* seq_ids, const int32_t* positions,
                    int num_tokens, const int32_t* block_tables, int max_blocks_per_seq,
                    int num_seqs, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    void* stream) {
  if (num_tokens < 0 || num_seqs <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PKV_ERR_INVALID_ARG, "kv_cache_append: non-positive size");
  if (num_tokens == 0) return ok();
  if (!k_pool || !v_pool || !k_new || !v_new || !seq_ids || !positions || !block_tables)
    return fail(PKV_ERR_INVALID_ARG, "kv_cache_append: null pointer");
  if ((int64_t)num_tokens * num_kv_heads * head_dim >= ((int64_t)1 << 31))
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_append: %d tokens x %d heads x %d too large",
                num_tokens, num_kv_heads, head_dim);
  const int es = elem_bytes(kv_dtype);
  if (es == 0) return fail(PKV_ERR_UNSUPPORTED, "kv_cache_append: kv_dtype %d", kv_dtype);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (validate_mode()) {
    std::vector<int32_t> sid, pos, tabs;
    if (!copy_ints(sid, seq_ids, num_tokens, st) || !copy_ints(pos, positions, num_tokens, st) ||
        !copy_ints(tabs, block_tables, (size_t)num_seqs * max_blocks_per_seq, st))
      return fail(PKV_ERR_LAUNCH, "kv_cache_append: validation copy failed");
    std::unordered_set<int64_t> slots;
    for (int i = 0; i < num_tokens; ++i) {
      if (sid[i] < 0 || sid[i] >= num_seqs)
        return fail(PKV_ERR_VALIDATION, "seq_ids[%d] = %d outside [0, %d)", i, sid[i], num_seqs);
      if (pos[i] < 0 || pos[i] / block_size >= max_blocks_per_seq)
        return fail(PKV_ERR_VALIDATION, "positions[%d] = %d outside the table", i, pos[i]);
      const int b = tabs[(size_t)sid[i] * max_blocks_per_seq + pos[i] / block_size];
      if (b < 0 || b >= num_blocks)
        return fail(PKV_ERR_VALIDATION, "token %d maps to block %d outside [0, %d)", i, b,
                    num_blocks);
      if (!slots.insert((int64_t)b * block_size + pos[i] % block_size).second)
        return fail(PKV_ERR_VALIDATION, "token %d writes a slot another token writes", i);
    }
  }
  pkv::AppendParams p{k_pool, v_pool, k_new, v_new, seq_ids, positions, block_tables,
                      num_tokens, max_blocks_per_seq, num_seqs, num_kv_heads, head_dim,
                      block_size, num_blocks};
  hipError_t e = timed("append", st, [&] { return pkv::launch_append(p, es, st); });
  if (e != hipSuccess) return launch_error(e, "kv_cache_append");
  return ok();
}

int cow_block_copy(void* k_pool, void* v_pool, int kv_dtype, const int32_t* src_blocks,
                   const int32_t* dst_blocks, const int32_t* num_tokens, int num_pairs,
                   int num_kv_heads, int head_dim, int block_size, int num_blocks, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "cow_block_copy: non-positive size");
  if (num_pairs == 0) return ok();
  if (!k_pool || !v_pool || !src_blocks || !dst_blocks)
    return fail(PKV_ERR_INVALID_ARG, "cow_block_copy: null pointer");
  const int es = elem_bytes(kv_dtype);
  if (es == 0) return fail(PKV_ERR_UNSUPPORTED, "cow_block_copy: kv_dtype %d", kv_dtype);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (validate_mode()) {
    std::vector<int32_t> src, dst, nt;
    if (!copy_ints(src, src_blocks, num_pairs, st) || !copy_ints(dst, dst_blocks, num_pairs, st) ||
        (num_tokens && !copy_ints(nt, num_tokens, num_pairs, st)))
      return fail(PKV_ERR_LAUNCH, "cow_block_copy: validation copy failed");
    std::unordered_set<int32_t> dsts;
    for (int i = 0; i < num_pairs; ++i) {
      if (src[i] < 0 || src[i] >= num_blocks || dst[i] < 0 || dst[i] >= num_blocks)
        return fail(PKV_ERR_VALIDATION, "pair %d: block outside [0, %d)", i, num_blocks);
      if (src[i] == dst[i]) return fail(PKV_ERR_VALIDATION, "pair %d: src == dst", i);
      if (!dsts.insert(dst[i]).second)
        return fail(PKV_ERR_VALIDATION, "pair %d: destination used twice", i);
      if (num_tokens && (nt[i] < 0 || nt[i] > block_size))
        return fail(PKV_ERR_VALIDATION, "pair %d: %d tokens", i, nt[i]);
    }
    for (int i = 0; i < num_pairs; ++i)
      if (dsts.count(src[i]))
        return fail(PKV_ERR_VALIDATION, "pair %d: source is another pair's destination", i);
  }
  pkv::CowParams p{k_pool, v_pool, src_blocks, dst_blocks, num_tokens, num_pairs,
                   num_kv_heads, head_dim, block_size, num_blocks};
  hipError_t e = timed("cow", st, [&] { return pkv::launch_cow(p, es, st); });
  if (e != hipSuccess) return launch_error(e, "cow_block_copy");
  return ok();
}

}  // extern "C"

namespace {

// Device address of a host buffer that the GPU may access directly (pinned with hipHostMalloc
// or registered), or nullptr. Pageable memory, device memory and unknown pointers give
// nullptr; the query's own error is cleared so that it does not surface at the next launch.
void* mapped_host_address(const void* p) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (a.type != hipMemoryTypeHost) return nullptr;
  return a.devicePointer;
}

// Shared body of kv_swap_out (to_host = true) and kv_swap_in.
int swap_impl(const char* fn, bool to_host, void* k_pool, void* v_pool, int kv_dtype,
              void* host_k, void* host_v, int num_host_blocks, const int32_t* src_blocks,
              const int32_t* dst_blocks, int num_pairs, int num_kv_heads, int head_dim,
              int block_size, int num_blocks, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || num_host_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: non-positive size", fn);
  if (!k_pool || !v_pool || !host_k || !host_v || !src_blocks || !dst_blocks)
    return fail(PKV_ERR_INVALID_ARG, "%s: null pointer", fn);
  const int es = elem_bytes(kv_dtype);
  if (es == 0) return fail(PKV_ERR_UNSUPPORTED, "%s: kv_dtype %d", fn, kv_dtype);
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * es;
  if (block_bytes % 16 != 0 || block_bytes / 16 >= ((int64_t)1 << 31))
    return fail(PKV_ERR_UNSUPPORTED, "%s: block of %lld bytes", fn, (long long)block_bytes);
  if ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool) |
       reinterpret_cast<uintptr_t>(host_k) | reinterpret_cast<uintptr_t>(host_v)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "%s: pools must be 16-byte aligned", fn);
  if (num_pairs == 0) return ok();
  void* hk = mapped_host_address(host_k);
  void* hv = mapped_host_address(host_v);
  if (!hk || !hv)
    return fail(PKV_ERR_INVALID_ARG,
                "%s: host_k / host_v must be pinned host memory mapped for the device", fn);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int src_count = to_host ? num_blocks : num_host_blocks;
  const int dst_count = to_host ? num_host_blocks : num_blocks;
  if (validate_mode()) {
    std::vector<int32_t> src, dst;
    if (!copy_ints(src, src_blocks, num_pairs, st) || !copy_ints(dst, dst_blocks, num_pairs, st))
      return fail(PKV_ERR_LAUNCH, "%s: validation copy failed", fn);
    std::unordered_set<int32_t> dsts;
    for (int i = 0; i < num_pairs; ++i) {
      if (src[i] < 0 || src[i] >= src_count)
        return fail(PKV_ERR_VALIDATION, "pair %d: source block %d outside [0, %d)", i, src[i],
                    src_count);
      if (dst[i] < 0 || dst[i] >= dst_count)
        return fail(PKV_ERR_VALIDATION, "pair %d: destination block %d outside [0, %d)", i,
                    dst[i], dst_count);
      if (!dsts.insert(dst[i]).second)
        return fail(PKV_ERR_VALIDATION, "pair %d: destination used twice", i);
    }
  }
  pkv::SwapParams p{};
  if (to_host) {
    p = {k_pool, v_pool, hk, hv, src_blocks, dst_blocks, num_pairs, src_count, dst_count,
         (int)(block_bytes / 16)};
  } else {
    p = {hk, hv, k_pool, v_pool, src_blocks, dst_blocks, num_pairs, src_count, dst_count,
         (int)(block_bytes / 16)};
  }
  const int cus = cu_count();
  hipError_t e = timed(to_host ? "swap_out" : "swap_in", st,
                       [&] { return pkv::launch_block_copy(p, cus, st); });
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

// Copy-engine swap: the device side through a contiguous staging buffer (one gather or scatter
// launch), the host side one DMA copy per pool between the staging buffer and a contiguous run
// of host blocks, so that no compute unit waits on the host link.
int swap_dma_impl(const char* fn, bool to_host, void* k_pool, void* v_pool, int kv_dtype,
                  void* host_k, void* host_v, int num_host_blocks, int host_block0,
                  const int32_t* device_blocks, int num_pairs, int num_kv_heads, int head_dim,
                  int block_size, int num_blocks, void* staging, size_t staging_bytes,
                  void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || num_host_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: non-positive size", fn);
  if (!k_pool || !v_pool || !host_k || !host_v || !device_blocks || !staging)
    return fail(PKV_ERR_INVALID_ARG, "%s: null pointer", fn);
  const int es = elem_bytes(kv_dtype);
  if (es == 0) return fail(PKV_ERR_UNSUPPORTED, "%s: kv_dtype %d", fn, kv_dtype);
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * es;
  if (block_bytes % 16 != 0 || block_bytes / 16 >= ((int64_t)1 << 31))
    return fail(PKV_ERR_UNSUPPORTED, "%s: block of %lld bytes", fn, (long long)block_bytes);
  if ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool) |
       reinterpret_cast<uintptr_t>(host_k) | reinterpret_cast<uintptr_t>(host_v) |
       reinterpret_cast<uintptr_t>(staging)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "%s: pools and staging must be 16-byte aligned", fn);
  if (host_block0 < 0 || (int64_t)host_block0 + num_pairs > num_host_blocks)
    return fail(PKV_ERR_INVALID_ARG, "%s: host blocks [%d, %lld) outside [0, %d)", fn,
                host_block0, (long long)host_block0 + num_pairs, num_host_blocks);
  const size_t run = (size_t)num_pairs * (size_t)block_bytes;
  if (staging_bytes < 2 * run)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "%s: staging %zu < %zu bytes", fn, staging_bytes,
                2 * run);
  if (num_pairs == 0) return ok();
  if (!mapped_host_address(host_k) || !mapped_host_address(host_v))
    return fail(PKV_ERR_INVALID_ARG, "%s: host_k / host_v must be pinned host memory", fn);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (validate_mode()) {
    std::vector<int32_t> ids;
    if (!copy_ints(ids, device_blocks, num_pairs, st))
      return fail(PKV_ERR_LAUNCH, "%s: validation copy failed", fn);
    std::unordered_set<int32_t> seen;
    for (int i = 0; i < num_pairs; ++i) {
      if (ids[i] < 0 || ids[i] >= num_blocks)
        return fail(PKV_ERR_VALIDATION, "pair %d: device block %d outside [0, %d)", i, ids[i],
                    num_blocks);
      if (!to_host && !seen.insert(ids[i]).second)
        return fail(PKV_ERR_VALIDATION, "pair %d: destination used twice", i);
    }
  }
  char* sk = reinterpret_cast<char*>(staging);
  char* sv = sk + run;
  char* hk = reinterpret_cast<char*>(host_k) + (size_t)host_block0 * (size_t)block_bytes;
  char* hv = reinterpret_cast<char*>(host_v) + (size_t)host_block0 * (size_t)block_bytes;
  const int cus = cu_count();
  const int units = (int)(block_bytes / 16);
  hipError_t e;
  if (to_host) {
    const pkv::SwapParams p{k_pool, v_pool, sk, sv, device_blocks, nullptr, num_pairs,
                            num_blocks, num_pairs, units};
    e = timed("swap_gather", st, [&] { return pkv::launch_block_copy(p, cus, st); });
    if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "%s: gather: %s", fn, hipGetErrorString(e));
    e = hipMemcpyAsync(hk, sk, run, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(hv, sv, run, hipMemcpyDeviceToHost, st);
    if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "%s: copy: %s", fn, hipGetErrorString(e));
  } else {
    e = hipMemcpyAsync(sk, hk, run, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(sv, hv, run, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "%s: copy: %s", fn, hipGetErrorString(e));
    const pkv::SwapParams p{sk, sv, k_pool, v_pool, nullptr, device_blocks, num_pairs,
                            num_pairs, num_blocks, units};
    e = timed("swap_scatter", st, [&] { return pkv::launch_block_copy(p, cus, st); });
    if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "%s: scatter: %s", fn, hipGetErrorString(e));
  }
  return ok();
}

// rows per KV head from which a workgroup's four wavefronts take four row tiles over the same
// tokens (extend_rows_shared)
constexpr int64_t kWideExtendRows = 128;

// Workspace of the shared-prefix call: the suffix decode's workspace, then the suffix lengths,
// the suffix rows' log-sum-exp, an fp32 suffix output (used when the output is 16-bit) and the
// prefix states of every chunk group.
struct SpLayout {
  size_t decode, suffix_lens, lse, o, m, l, acc, total;
  int chunk_groups, steps_per_chunk;
  bool wide;
};

// Prefix states: at least 128 rows per KV head over more than kWidePrefixTokens take the kernel
// whose workgroups share each step's keys and values among four 32-row tiles, with chunk groups
// enough for kWidePrefixWgPerCu workgroups per CU; shorter prefixes the row-state kernel, whose
// four wavefronts split one 32-row tile's tokens. Up to 4096 tokens the row-state kernel leaves
// one state per row for the merge to read (four wavefronts of at most 32 steps); the wide
// kernel's chunk groups (eight at 1024 rows per KV head) cost the merge about 1 us each, which
// its faster steps repay only beyond that.
constexpr int kWidePrefixTokens = 4096;
constexpr int kWidePrefixWgPerCu = 2;

SpLayout sp_layout(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int n,
                   int prefix_len) {
  const int G = num_q_heads / num_kv_heads;
  SpLayout L;
  L.wide = (int64_t)num_seqs * G >= kWideExtendRows && prefix_len > kWidePrefixTokens;
  if (L.wide) {
    pkv::wide_row_plan((int64_t)num_kv_heads * pkv::wide_row_groups((int64_t)num_seqs * G),
                       prefix_len, kWidePrefixWgPerCu * cu_count(), &L.chunk_groups);
    L.steps_per_chunk = 0;
  } else {
    pkv::row_state_plan((int64_t)num_kv_heads * pkv::row_groups((int64_t)num_seqs * G),
                        prefix_len, cu_count(), &L.chunk_groups, &L.steps_per_chunk);
  }
  const size_t SH = (size_t)num_seqs * num_q_heads;
  L.decode = ws_layout(num_seqs, G, head_dim, n).total;
  L.suffix_lens = align256(L.decode);
  L.lse = L.suffix_lens + align256((size_t)num_seqs * sizeof(int32_t));
  L.o = L.lse + align256(SH * sizeof(float));
  L.m = L.o + align256(SH * head_dim * sizeof(float));
  L.l = L.m + align256((size_t)L.chunk_groups * SH * sizeof(float));
  L.acc = L.l + align256((size_t)L.chunk_groups * SH * sizeof(float));
  L.total = L.acc + align256((size_t)L.chunk_groups * SH * head_dim * sizeof(float));
  return L;
}

}  // namespace

extern "C" {

size_t pkv_shared_prefix_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, int num_workers, int prefix_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_q_heads % num_kv_heads != 0 || num_workers < 0 || prefix_len <= 0)
    return 0;
  return sp_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, choose_workers(num_workers),
                   prefix_len)
      .total;
}

int paged_attn_decode_shared_prefix(void* out, int out_dtype, const void* q, const void* k_pool,
                                    const void* v_pool, int kv_dtype,
                                    const int32_t* prefix_blocks, int prefix_len,
                                    const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* context_lens, int max_context_len,
                                    int num_seqs, int num_q_heads, int num_kv_heads,
                                    int head_dim, int block_size, int num_blocks, float scale,
                                    int num_workers, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  const char* fn = "paged_attn_decode_shared_prefix";
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || max_context_len < 0 || num_workers < 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: non-positive size", fn);
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !prefix_blocks || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: kv_dtype %d (fp16 or bf16 caches)", fn, kv_dtype);
  if (!(out_dtype == PKV_F32 || out_dtype == kv_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "%s: out_dtype %d with kv_dtype %d", fn, out_dtype,
                kv_dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, head_dim);
  if (block_size != 16 && block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "%s: block_size %d (16 or 32)", fn, block_size);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: %d query heads not a multiple of %d KV heads", fn,
                num_q_heads, num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  // the suffix decode and the merge take every sharer in one launch (checked before anything
  // is enqueued)
  if (num_seqs > pkv::kMaxSeqsPerCall)
    return fail(PKV_ERR_UNSUPPORTED, "%s: %d sequences (at most %d per call)", fn, num_seqs,
                pkv::kMaxSeqsPerCall);
  if (num_workers > (1 << 20))
    return fail(PKV_ERR_INVALID_ARG, "%s: num_workers %d", fn, num_workers);
  if (prefix_len <= 0 || prefix_len % block_size != 0 || prefix_len > max_context_len)
    return fail(PKV_ERR_INVALID_ARG,
                "%s: prefix_len %d must be a positive multiple of %d, at most %d", fn,
                prefix_len, block_size, max_context_len);
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_ERR_INVALID_ARG, "%s: max_context_len %d exceeds table capacity %d x %d",
                fn, max_context_len, max_blocks_per_seq, block_size);
  // the workspace holds the partial slots of the automatic worker count's upper bound; the
  // suffix decode itself picks its count as the plain decode does (every worker resident)
  const SpLayout sl = sp_layout(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                choose_workers(num_workers), prefix_len);
  if (!workspace || workspace_bytes < sl.total)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn,
                workspace_bytes, sl.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(PKV_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", fn);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int nb = prefix_len / block_size;

  if (validate_mode()) {
    std::vector<int32_t> lens, tabs, pre;
    if (!copy_ints(lens, context_lens, num_seqs, st) || !copy_ints(pre, prefix_blocks, nb, st) ||
        !copy_ints(tabs, block_tables, (size_t)num_seqs * max_blocks_per_seq, st))
      return fail(PKV_ERR_LAUNCH, "%s: validation copy failed", fn);
    for (int j = 0; j < nb; ++j)
      if (pre[j] < 0 || pre[j] >= num_blocks)
        return fail(PKV_ERR_VALIDATION, "prefix_blocks[%d] = %d outside [0, %d)", j, pre[j],
                    num_blocks);
    for (int s = 0; s < num_seqs; ++s) {
      if (lens[s] < prefix_len || lens[s] > max_context_len)
        return fail(PKV_ERR_VALIDATION, "context_lens[%d] = %d outside [%d, %d]", s, lens[s],
                    prefix_len, max_context_len);
      const int32_t* row = tabs.data() + (size_t)s * max_blocks_per_seq;
      for (int j = 0; j < nb; ++j)
        if (row[j] != pre[j])
          return fail(PKV_ERR_VALIDATION, "block_tables[%d][%d] = %d is not prefix block %d", s,
                      j, row[j], pre[j]);
      const int nbs = (lens[s] + block_size - 1) / block_size;
      for (int j = nb; j < nbs; ++j)
        if (row[j] < 0 || row[j] >= num_blocks)
          return fail(PKV_ERR_VALIDATION, "block_tables[%d][%d] = %d outside [0, %d)", s, j,
                      row[j], num_blocks);
    }
  }

  char* ws = reinterpret_cast<char*>(workspace);
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)head_dim);
  int32_t* suffix_lens = reinterpret_cast<int32_t*>(ws + sl.suffix_lens);
  float* lse = reinterpret_cast<float*>(ws + sl.lse);
  float* o_suffix = out_dtype == PKV_F32 ? reinterpret_cast<float*>(out)
                                         : reinterpret_cast<float*>(ws + sl.o);
  float* st_m = reinterpret_cast<float*>(ws + sl.m);
  float* st_l = reinterpret_cast<float*>(ws + sl.l);
  float* st_acc = reinterpret_cast<float*>(ws + sl.acc);

  pkv::RowStateParams pp{};
  pp.q = q;
  pp.k_pool = k_pool;
  pp.v_pool = v_pool;
  pp.lens = context_lens;
  pp.prefix_blocks = prefix_blocks;
  pp.suffix_lens = suffix_lens;
  pp.prefix_len = prefix_len;
  pp.st_m = st_m;
  pp.st_l = st_l;
  pp.st_acc = st_acc;
  pp.state_rows = (size_t)num_seqs * num_q_heads;
  pp.num_seqs = num_seqs;
  pp.num_q_heads = num_q_heads;
  pp.num_kv_heads = num_kv_heads;
  pp.num_blocks = num_blocks;
  pp.chunk_groups = sl.chunk_groups;
  pp.steps_per_chunk = sl.steps_per_chunk;
  pp.scale_log2 = sc * 1.4426950408889634f;
  hipError_t e = timed("prefix_states", st, [&] {
    return sl.wide ? pkv::launch_wide_prefix_states(pp, kv_dtype, head_dim, block_size, st)
                   : pkv::launch_row_states(pp, kv_dtype, head_dim, block_size, st);
  });
  if (e != hipSuccess) return fail(PKV_ERR_LAUNCH, "%s: prefix kernel: %s", fn,
                                   hipGetErrorString(e));
  // the suffix: the same tables past the prefix entries (row stride unchanged), the lengths
  // the prefix kernel wrote; the merge folds each row's suffix state with its prefix states
  const PrefixFold pf{lse, out, out_dtype == PKV_F32 ? 1 : 0, st_m, st_l, st_acc,
                      sl.chunk_groups};
  const int rc = decode_impl(fn, o_suffix, PKV_F32, q, k_pool, v_pool, kv_dtype, nullptr,
                             nullptr, block_tables + nb, max_blocks_per_seq, suffix_lens,
                             max_context_len - prefix_len, num_seqs, num_q_heads, num_kv_heads,
                             head_dim, block_size, num_blocks, scale, num_workers, workspace,
                             sl.decode, stream, &pf);
  if (rc != PKV_OK) return rc;
  return ok();
}

}  // extern "C"

namespace {

// Workspace of paged_attn_extend: the row states of every chunk group. Runs of new tokens whose
// rows per KV head reach 128 (max_query_len * G) take the kernel with workgroup-shared key/value
// tiles; shorter runs (speculative verification) the row-state kernel, whose four wavefronts
// split a 32-row group's tokens.
struct ExtLayout {
  size_t m, l, acc, total;
  int chunk_groups, steps_per_chunk, max_row_groups;
  bool wide;
};

ExtLayout ext_layout(int num_seqs, int num_query_tokens, int num_q_heads, int num_kv_heads,
                     int head_dim, int max_query_len, int max_context_len) {
  const int G = num_q_heads / num_kv_heads;
  ExtLayout L;
  L.wide = (int64_t)max_query_len * G >= kWideExtendRows;
  if (L.wide) {
    L.max_row_groups = (int)pkv::wide_row_groups((int64_t)max_query_len * G);
    pkv::wide_row_plan((int64_t)num_seqs * num_kv_heads * L.max_row_groups, max_context_len,
                       cu_count(), &L.chunk_groups);
    L.steps_per_chunk = 0;
  } else {
    L.max_row_groups = (int)pkv::row_groups((int64_t)max_query_len * G);
    pkv::row_state_plan((int64_t)num_seqs * num_kv_heads * L.max_row_groups, max_context_len,
                        cu_count(), &L.chunk_groups, &L.steps_per_chunk);
  }
  const size_t rows = (size_t)num_query_tokens * num_q_heads;
  L.m = 0;
  L.l = align256((size_t)L.chunk_groups * rows * sizeof(float));
  L.acc = L.l + align256((size_t)L.chunk_groups * rows * sizeof(float));
  L.total = L.acc + align256((size_t)L.chunk_groups * rows * head_dim * sizeof(float));
  return L;
}

}  // namespace

extern "C" {

size_t pkv_extend_workspace_size(int num_seqs, int num_query_tokens, int num_q_heads,
                                 int num_kv_heads, int head_dim, int max_query_len,
                                 int max_context_len) {
  if (num_seqs <= 0 || num_query_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || num_q_heads % num_kv_heads != 0 || max_query_len <= 0 ||
      max_context_len <= 0)
    return 0;
  return ext_layout(num_seqs, num_query_tokens, num_q_heads, num_kv_heads, head_dim,
                    max_query_len, max_context_len)
      .total;
}

int paged_attn_extend(void* out, int out_dtype, const void* q, const int32_t* query_start,
                      int num_query_tokens, int max_query_len, const void* k_pool,
                      const void* v_pool, int kv_dtype, const int32_t* block_tables,
                      int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, float scale, void* workspace,
                      size_t workspace_bytes, void* stream) {
  const char* fn = "paged_attn_extend";
  if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: negative or non-positive size", fn);
  if (num_seqs == 0 || num_query_tokens == 0) return ok();
  if (!out || !q || !query_start || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: kv_dtype %d (fp16 or bf16 caches)", fn, kv_dtype);
  if (!(out_dtype == PKV_F32 || out_dtype == kv_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "%s: out_dtype %d with kv_dtype %d", fn, out_dtype,
                kv_dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, head_dim);
  if (block_size != 16 && block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "%s: block_size %d (16 or 32)", fn, block_size);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: %d query heads not a multiple of %d KV heads", fn,
                num_q_heads, num_kv_heads);
  if (max_query_len == 0 || max_query_len > num_query_tokens || max_context_len == 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: max_query_len %d (1 to %d), max_context_len %d", fn,
                max_query_len, num_query_tokens, max_context_len);
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_ERR_INVALID_ARG, "%s: max_context_len %d exceeds table capacity %d x %d",
                fn, max_context_len, max_blocks_per_seq, block_size);
  const ExtLayout el = ext_layout(num_seqs, num_query_tokens, num_q_heads, num_kv_heads,
                                  head_dim, max_query_len, max_context_len);
  if (!workspace || workspace_bytes < el.total)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn,
                workspace_bytes, el.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(PKV_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", fn);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  if (validate_mode()) {
    std::vector<int32_t> qs, lens, tabs;
    if (!copy_ints(qs, query_start, (size_t)num_seqs + 1, st) ||
        !copy_ints(lens, context_lens, num_seqs, st) ||
        !copy_ints(tabs, block_tables, (size_t)num_seqs * max_blocks_per_seq, st))
      return fail(PKV_ERR_LAUNCH, "%s: validation copy failed", fn);
    if (qs[0] != 0 || qs[num_seqs] != num_query_tokens)
      return fail(PKV_ERR_VALIDATION, "query_start must run from 0 to %d", num_query_tokens);
    for (int s = 0; s < num_seqs; ++s) {
      const int n = qs[s + 1] - qs[s];
      if (n < 0 || n > max_query_len)
        return fail(PKV_ERR_VALIDATION, "sequence %d: %d query tokens (0 to %d)", s, n,
                    max_query_len);
      if (lens[s] < n || lens[s] > max_context_len)
        return fail(PKV_ERR_VALIDATION, "context_lens[%d] = %d outside [%d, %d]", s, lens[s], n,
                    max_context_len);
      const int nbs = (lens[s] + block_size - 1) / block_size;
      for (int j = 0; j < nbs; ++j) {
        const int b = tabs[(size_t)s * max_blocks_per_seq + j];
        if (b < 0 || b >= num_blocks)
          return fail(PKV_ERR_VALIDATION, "block_tables[%d][%d] = %d outside [0, %d)", s, j, b,
                      num_blocks);
      }
    }
  }

  char* ws = reinterpret_cast<char*>(workspace);
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)head_dim);
  pkv::RowStateParams rp{};
  rp.q = q;
  rp.k_pool = k_pool;
  rp.v_pool = v_pool;
  rp.lens = context_lens;
  rp.query_start = query_start;
  rp.tables = block_tables;
  rp.max_blocks = max_blocks_per_seq;
  rp.max_row_groups = el.max_row_groups;
  rp.num_query_tokens = num_query_tokens;
  rp.st_m = reinterpret_cast<float*>(ws + el.m);
  rp.st_l = reinterpret_cast<float*>(ws + el.l);
  rp.st_acc = reinterpret_cast<float*>(ws + el.acc);
  rp.state_rows = (size_t)num_query_tokens * num_q_heads;
  rp.num_seqs = num_seqs;
  rp.num_q_heads = num_q_heads;
  rp.num_kv_heads = num_kv_heads;
  rp.num_blocks = num_blocks;
  rp.chunk_groups = el.chunk_groups;
  rp.steps_per_chunk = el.steps_per_chunk;
  rp.scale_log2 = sc * 1.4426950408889634f;
  // one chunk group: each workgroup's merged state is its rows' whole softmax, normalised and
  // written straight to `out` (no finish kernel)
  const bool direct = el.chunk_groups == 1;
  rp.out = direct ? out : nullptr;
  rp.out_f32 = out_dtype == PKV_F32 ? 1 : 0;
  hipError_t e = timed("extend_states", st, [&] {
    return el.wide ? pkv::launch_extend_rows_shared(rp, kv_dtype, head_dim, block_size, st)
                   : pkv::launch_row_states(rp, kv_dtype, head_dim, block_size, st);
  });
  if (e != hipSuccess)
    return fail(PKV_ERR_LAUNCH, "%s: states kernel: %s", fn, hipGetErrorString(e));
  if (direct) return ok();
  pkv::ExtendFinishParams fp{out, rp.st_m, rp.st_l, rp.st_acc, rp.state_rows, el.chunk_groups,
                             out_dtype == PKV_F32 ? 1 : 0};
  e = timed("extend_finish", st,
            [&] { return pkv::launch_extend_finish(fp, kv_dtype, head_dim, st); });
  if (e != hipSuccess)
    return fail(PKV_ERR_LAUNCH, "%s: finish kernel: %s", fn, hipGetErrorString(e));
  return ok();
}

int kv_swap_out(const void* k_pool, const void* v_pool, int kv_dtype, void* host_k,
                void* host_v, int num_host_blocks, const int32_t* device_blocks,
                const int32_t* host_blocks, int num_pairs, int num_kv_heads, int head_dim,
                int block_size, int num_blocks, void* stream) {
  return swap_impl("kv_swap_out", true, const_cast<void*>(k_pool), const_cast<void*>(v_pool),
                   kv_dtype, host_k, host_v, num_host_blocks, device_blocks, host_blocks,
                   num_pairs, num_kv_heads, head_dim, block_size, num_blocks, stream);
}

int kv_swap_in(void* k_pool, void* v_pool, int kv_dtype, const void* host_k, const void* host_v,
               int num_host_blocks, const int32_t* host_blocks, const int32_t* device_blocks,
               int num_pairs, int num_kv_heads, int head_dim, int block_size, int num_blocks,
               void* stream) {
  return swap_impl("kv_swap_in", false, k_pool, v_pool, kv_dtype, const_cast<void*>(host_k),
                   const_cast<void*>(host_v), num_host_blocks, host_blocks, device_blocks,
                   num_pairs, num_kv_heads, head_dim, block_size, num_blocks, stream);
}

size_t pkv_swap_staging_size(int num_pairs, int num_kv_heads, int head_dim, int block_size,
                             int kv_dtype) {
  const int es = elem_bytes(kv_dtype);
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || es == 0)
    return 0;
  return 2 * (size_t)num_pairs * (size_t)num_kv_heads * block_size * head_dim * es;
}

int kv_swap_out_dma(const void* k_pool, const void* v_pool, int kv_dtype, void* host_k,
                    void* host_v, int num_host_blocks, const int32_t* device_blocks,
                    int host_block0, int num_pairs, int num_kv_heads, int head_dim,
                    int block_size, int num_blocks, void* staging, size_t staging_bytes,
                    void* stream) {
  return swap_dma_impl("kv_swap_out_dma", true, const_cast<void*>(k_pool),
                       const_cast<void*>(v_pool), kv_dtype, host_k, host_v, num_host_blocks,
                       host_block0, device_blocks, num_pairs, num_kv_heads, head_dim,
                       block_size, num_blocks, staging, staging_bytes, stream);
}

int kv_swap_in_dma(void* k_pool, void* v_pool, int kv_dtype, const void* host_k,
                   const void* host_v, int num_host_blocks, int host_block0,
                   const int32_t* device_blocks, int num_pairs, int num_kv_heads, int head_dim,
                   int block_size, int num_blocks, void* staging, size_t staging_bytes,
                   void* stream) {
  return swap_dma_impl("kv_swap_in_dma", false, k_pool, v_pool, kv_dtype,
                       const_cast<void*>(host_k), const_cast<void*>(host_v), num_host_blocks,
                       host_block0, device_blocks, num_pairs, num_kv_heads, head_dim,
                       block_size, num_blocks, staging, staging_bytes, stream);
}

int pkv_set_validate(int on) {
  g_validate = on ? 1 : 0;
  return ok();
}

int pkv_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto& r : g_recs) {
    g_spare.push_back(r.start);
    g_spare.push_back(r.stop);
  }
  g_recs.clear();
  g_seen.clear();
  g_timing = on > 0;
  g_timing_every = on > 0 ? on : 1;
  return ok();
}

int pkv_timing_query(const char* name, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(PKV_ERR_INVALID_ARG, "pkv_timing_query: null pointer");
  std::lock_guard<std::mutex> lk(g_tmu);
  double tot = 0.0;
  int64_t n = 0;
  for (auto& r : g_recs) {
    if (name && *name && !std::strstr(r.name, name)) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess)
      return fail(PKV_ERR_LAUNCH, "pkv_timing_query: event wait failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      return fail(PKV_ERR_LAUNCH, "pkv_timing_query: elapsed time failed");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return ok();
}

int pkv_mfma_rate_probe(int workgroups, int iters, float* sink, void* stream) {
  if (!sink) return fail(PKV_ERR_INVALID_ARG, "pkv_mfma_rate_probe: null pointer");
  if (workgroups <= 0 || iters <= 0 || workgroups > (1 << 20))
    return fail(PKV_ERR_INVALID_ARG, "pkv_mfma_rate_probe: %d workgroups, %d rounds",
                workgroups, iters);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = timed("mfma_rate", st,
                       [&] { return pkv::launch_mfma_rate(workgroups, iters, sink, st); });
  if (e != hipSuccess) return launch_error(e, "pkv_mfma_rate_probe");
  return ok();
}

int pkv_stream_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return fail(PKV_ERR_INVALID_ARG, "pkv_stream_read_probe: null pointer");
  if (bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15))
    return fail(PKV_ERR_INVALID_ARG, "pkv_stream_read_probe: %zu bytes / alignment", bytes);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int cus = cu_count();
  hipError_t e = timed("stream_read", st,
                       [&] { return pkv::launch_stream_read(src, bytes, sink, cus, st); });
  if (e != hipSuccess) return launch_error(e, "pkv_stream_read_probe");
  return ok();
}

}  // extern "C"
