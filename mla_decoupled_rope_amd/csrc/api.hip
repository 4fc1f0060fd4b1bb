// C-ABI host layer of libmla: argument checks, the decode split plan, and
// the kernel launches.  Nothing here allocates device memory or synchronises.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <queue>
#include <string>
#include <vector>

#include "common.hpp"
#include "mla.h"

namespace {

thread_local std::string g_err;

mla_status fail(mla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

mla_status hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MLA_TRY(expr)                   \
  do {                                  \
    const mla_status st_ = (expr);      \
    if (st_ != MLA_OK) return st_;      \
  } while (0)

// Cache lines and CUs: the plan is a pure function of the lengths and these
// constants, so the same batch always splits the same way on any device.
constexpr int kPlanCUs = 256;
constexpr size_t kWsAlign = 256;

// The rotated query carries the position part's scale relative to the
// content part's, so one softmax_scale on the summed score gives both.
double position_ratio(const mla_dims* d) {
  return static_cast<double>(d->position_scale) / static_cast<double>(d->softmax_scale);
}

mla_status check_dims(const mla_dims* d) {
  if (d == nullptr) return fail(MLA_ERR_INVALID_ARG, "dims is NULL");
  if (d->n_heads <= 0 || d->d_head <= 0 || d->d_v <= 0 || d->d_latent <= 0 || d->d_rope <= 0)
    return fail(MLA_ERR_INVALID_ARG, "every dimension must be positive (n_heads=%d d_head=%d d_v=%d d_latent=%d d_rope=%d)",
                d->n_heads, d->d_head, d->d_v, d->d_latent, d->d_rope);
  if (d->d_rope % 2 != 0) return fail(MLA_ERR_INVALID_ARG, "d_rope must be even (got %d)", d->d_rope);
  if (d->d_rope > 128) return fail(MLA_ERR_UNSUPPORTED, "d_rope > 128 is not supported (got %d)", d->d_rope);
  if (d->page_size != mla::kPage) return fail(MLA_ERR_UNSUPPORTED, "page_size must be 64 (got %d)", d->page_size);
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (d->work_dtype != MLA_F32 && d->work_dtype != MLA_BF16)
    return fail(MLA_ERR_INVALID_ARG, "unknown work_dtype %d", d->work_dtype);
  if (d->dtype == MLA_F32 && d->work_dtype != MLA_F32)
    return fail(MLA_ERR_INVALID_ARG, "float32 inputs need the float32 working precision");
  if (!(std::isfinite(d->softmax_scale) && d->softmax_scale > 0.f))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and positive");
  if (!(std::isfinite(d->position_scale) && d->position_scale > 0.f))
    return fail(MLA_ERR_INVALID_ARG, "position_scale must be finite and positive");
  if (!(std::isfinite(d->rope_base) && d->rope_base > 0.0))
    return fail(MLA_ERR_INVALID_ARG, "rope_base must be finite and positive");
  return MLA_OK;
}

mla_status check_attn_shape(const mla_dims* d) {
  if (d->dtype == MLA_BF16) {
    const bool dsv2 = d->n_heads == 128 && d->d_latent == 512 && d->d_rope == 64;
    const bool tiny = d->n_heads == 16 && d->d_latent == 256 && d->d_rope == 32;
    if (d->work_dtype == MLA_F32 && d->d_latent + d->d_rope > 288)
      return fail(MLA_ERR_UNSUPPORTED, "the float32 working precision needs d_latent + d_rope <= 288");
    if (!dsv2 && !tiny)
      return fail(MLA_ERR_UNSUPPORTED,
                  "bf16 attention supports (n_heads, d_latent, d_rope) = (128, 512, 64) or (16, 256, 32); got (%d, %d, %d)",
                  d->n_heads, d->d_latent, d->d_rope);
  } else {
    if (d->n_heads > 1024 || d->d_latent > 1024 || d->d_latent + d->d_rope > 1152)
      return fail(MLA_ERR_UNSUPPORTED, "float32 attention needs n_heads <= 1024, d_latent <= 1024, d_latent + d_rope <= 1152");
  }
  return MLA_OK;
}

mla_status check_cache(const mla_paged_cache* c) {
  if (c == nullptr) return fail(MLA_ERR_INVALID_ARG, "cache is NULL");
  if (c->num_pages < 0 || c->num_seqs < 0 || c->max_pages_per_seq <= 0)
    return fail(MLA_ERR_INVALID_ARG, "cache sizes must be non-negative (num_pages=%lld num_seqs=%d max_pages_per_seq=%d)",
                static_cast<long long>(c->num_pages), c->num_seqs, c->max_pages_per_seq);
  if (c->num_pages > 0 && c->data == nullptr) return fail(MLA_ERR_INVALID_ARG, "cache->data is NULL");
  if (c->num_seqs > 0 && c->block_table == nullptr) return fail(MLA_ERR_INVALID_ARG, "cache->block_table is NULL");
  if (c->num_pages > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "more than 2^31 - 1 pages");
  return MLA_OK;
}

struct Plan {
  int split_pages = 1;
  int n_full = 0;
  int64_t n_items = 0;  // (sequence, split) pairs = partial slots
  bool needs_merge = false;
};

int env_split_pages() {
  const char* e = std::getenv("MLA_DECODE_SPLIT_PAGES");
  if (e == nullptr || *e == '\0') return 0;
  const long v = std::strtol(e, nullptr, 10);
  return v > 0 && v < (1 << 30) ? static_cast<int>(v) : 0;
}

// Makespan of the item list under greedy list scheduling on `workers`
// identical workers: first the full splits of split sequences, then the
// single-item sequences of exactly L pages, then the remainders.  The first
// group all cost the same, so greedy placement deals them out evenly: r
// workers end at `hi`, the others at `lo`.  The other two groups hold at most
// one item per sequence; a heap tracks only the workers they have touched,
// while untouched ones are counted per level.
double simulate(const std::vector<int>& pages, int L, int workers, double item_cost, double partial_cost) {
  int64_t n_split = 0;
  for (int pg : pages)
    if (pg > L) n_split += pg / L;
  const int64_t q = n_split / workers, r = n_split % workers;
  const double lo = static_cast<double>(q) * (L + item_cost + partial_cost);
  const double hi = r > 0 ? lo + (L + item_cost + partial_cost) : lo;
  int64_t n_lo = workers - r, n_hi = r;
  double makespan = n_hi > 0 ? hi : lo;
  std::priority_queue<double, std::vector<double>, std::greater<double>> touched;
  auto run = [&](double cost) {
    // the least loaded worker: an untouched one at lo, else the lesser of hi and the heap's top
    double t;
    if (n_lo > 0) {
      t = lo;
      --n_lo;
    } else if (n_hi > 0 && (touched.empty() || hi <= touched.top())) {
      t = hi;
      --n_hi;
    } else {
      t = touched.top();
      touched.pop();
    }
    t += cost;
    touched.push(t);
    makespan = std::max(makespan, t);
  };
  for (int pg : pages)
    if (pg == L) run(L + item_cost);
  for (int pg : pages)
    if (pg % L) run(pg % L + item_cost + (pg > L ? partial_cost : 0.0));
  return makespan;
}

// Split partials of the shared-key decode at d_c = 512 in bf16 working
// precision are float16 with a power-of-two scale per 128-column quarter of a
// row (half the bytes of float32 at 2^-11 relative rounding); every other
// decode keeps float32 partials.
bool half_partials(const mla_dims* d) {
  return d->dtype == MLA_BF16 && d->work_dtype == MLA_BF16 && d->d_latent == 512 && d->d_rope == 64;
}

Plan compute_plan(const mla_dims* d, const std::vector<int>& pages, int env) {
  Plan p;
  const int batch = static_cast<int>(pages.size());
  int64_t total = 0;
  int max_pages = 1;
  for (int pg : pages) {
    total += pg;
    max_pages = std::max(max_pages, pg);
  }
  int L = env;
  if (L == 0) {
    const int row = d->d_latent + d->d_rope;
    const int wg_per_cu = row > 288 ? 1 : 2;
    const int workers = kPlanCUs * wg_per_cu;
    const double page_bytes = 64.0 * row * 2.0;
    const double elt = half_partials(d) ? 2.0 : 4.0;  // bytes of a stored partial element
    const double partial_cost = 2.0 * d->n_heads * (d->d_latent * elt + 4.0) / page_bytes;  // write + merge read
    const double item_cost = 1.0;
    double best = -1.0;
    L = max_pages;
    std::vector<int> cands = {max_pages};
    for (int k = 1; k <= 16; ++k) {
      const int64_t c = (total + static_cast<int64_t>(workers) * k - 1) / (static_cast<int64_t>(workers) * k);
      cands.push_back(static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(c, max_pages))));
    }
    std::sort(cands.begin(), cands.end());
    cands.erase(std::unique(cands.begin(), cands.end()), cands.end());
    for (int c : cands) {
      const double m = simulate(pages, c, workers, item_cost, partial_cost);
      if (best < 0 || m < best - 1e-9 || (std::fabs(m - best) <= 1e-9 && c > L)) {
        best = m;
        L = c;
      }
    }
  }
  p.split_pages = L;
  int64_t n_full = 0, n_rem = 0;
  for (int b = 0; b < batch; ++b) {
    n_full += pages[b] / L;
    n_rem += (pages[b] % L) != 0;
    const int ns = pages[b] / L + ((pages[b] % L) != 0);
    if (ns != 1) p.needs_merge = true;
  }
  p.n_full = static_cast<int>(n_full);
  p.n_items = n_full + n_rem;
  return p;
}

// A serving loop asks for the same plan twice per step (workspace size, then
// decode), and the plan changes only when a sequence enters a new page: keep
// the last plan of each host thread, keyed by everything compute_plan reads.
Plan make_plan(const mla_dims* d, int batch, const int32_t* lens) {
  struct Entry {
    int n_heads = -1, d_latent = -1, d_rope = -1, env = -1;
    std::vector<int> pages;
    Plan plan;
  };
  thread_local Entry last;
  thread_local std::vector<int> pages;
  pages.resize(batch);
  for (int b = 0; b < batch; ++b) pages[b] = (std::max(lens[b], 0) + mla::kPage - 1) / mla::kPage;
  const int env = env_split_pages();
  if (last.n_heads == d->n_heads && last.d_latent == d->d_latent && last.d_rope == d->d_rope && last.env == env &&
      last.pages == pages)
    return last.plan;
  last.plan = compute_plan(d, pages, env);
  last.n_heads = d->n_heads; last.d_latent = d->d_latent; last.d_rope = d->d_rope; last.env = env;
  last.pages = pages;
  return last.plan;
}

// Workspace: normalised obar partials [n_items, H, d_latent] (float32, or
// float16 with int32 quarter exponents [n_items, H, d_latent / 128] after
// them), then lse [n_items, H] float32, each part at a 256-byte aligned offset.
size_t align_ws(size_t n) { return (n + kWsAlign - 1) / kWsAlign * kWsAlign; }

size_t partial_bytes(const mla_dims* d, const Plan& p) {
  const size_t rows = static_cast<size_t>(p.n_items) * d->n_heads;
  if (half_partials(d)) return align_ws(rows * d->d_latent * 2) + align_ws(rows * (d->d_latent / 128) * 4);
  return align_ws(rows * d->d_latent * sizeof(float));
}

size_t workspace_bytes(const mla_dims* d, const Plan& p) {
  if (d->dtype != MLA_BF16 || !p.needs_merge || p.n_items == 0) return 0;
  return partial_bytes(d, p) + static_cast<size_t>(p.n_items) * d->n_heads * sizeof(float);
}

// Workspace of mla_decode_proj: a partial slot for every work item, split or
// not (the fused merge reads only partials), laid out as workspace_bytes';
// on float32 caches the float32 obar [batch, H, d_latent] instead.
size_t proj_workspace_bytes(const mla_dims* d, const Plan& p, int32_t batch) {
  if (d->dtype == MLA_F32) return align_ws(static_cast<size_t>(batch) * d->n_heads * d->d_latent * sizeof(float));
  if (p.n_items == 0) return 0;
  return partial_bytes(d, p) + static_cast<size_t>(p.n_items) * d->n_heads * sizeof(float);
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Debug mode: with MLA_DEBUG_VALIDATE=1 in the environment, every call that
// reads or writes the paged cache first checks on the device the block-table
// entries and cache rows it will use, and that the device lengths are the host
// copies it planned with; it synchronises the stream for that, and launches
// nothing if the check fails.
bool debug_validate() {
  const char* e = std::getenv("MLA_DEBUG_VALIDATE");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

mla_status device_check(const mla_paged_cache* cache, int32_t batch, const int32_t* seq_lens,
                        const int32_t* seq_lens_host, const int32_t* cu_q, const int32_t* q_start,
                        const int32_t* cu_q_host, const int32_t* q_start_host, const int32_t* kv_seq,
                        const int32_t* kv_pos, int64_t n_kv, void* stream) {
  const mla::CheckParams c{cache->block_table, cache->num_seqs, cache->max_pages_per_seq, cache->num_pages, batch,
                           seq_lens, cu_q, q_start, kv_seq, kv_pos, n_kv};
  int32_t rec[6] = {};
  const hipError_t e = mla::run_check(c, rec, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "MLA_DEBUG_VALIDATE check");
  switch (rec[0]) {
    case mla::kCheckPage:
      return fail(MLA_ERR_INVALID_ARG, "MLA_DEBUG_VALIDATE: block_table[%d][%d] = %d is not a page of the cache "
                  "(0 .. %lld)", rec[1], rec[2], rec[3], static_cast<long long>(cache->num_pages) - 1);
    case mla::kCheckLength:
      return fail(MLA_ERR_INVALID_ARG, "MLA_DEBUG_VALIDATE: sequence %d reaches %d tokens on the device, beyond its "
                  "block table", rec[1], rec[2]);
    case mla::kCheckRow:
      return fail(MLA_ERR_INVALID_ARG, "MLA_DEBUG_VALIDATE: cache row %d (sequence %d, position %d) has no page in "
                  "the block table", rec[1], rec[2], rec[3]);
    default:
      break;
  }
  unsigned sum = 0, hash = 0;
  for (int b = 0; b < batch; ++b) {
    const int t = cu_q_host != nullptr ? q_start_host[b] + (cu_q_host[b + 1] - cu_q_host[b]) : seq_lens_host[b];
    sum += static_cast<unsigned>(t);
    hash ^= (static_cast<unsigned>(t) * 2654435761u) ^ static_cast<unsigned>(b);
  }
  if (static_cast<int32_t>(sum) != rec[4] || static_cast<int32_t>(hash) != rec[5])
    return fail(MLA_ERR_INVALID_ARG, "MLA_DEBUG_VALIDATE: the device lengths differ from their host copies");
  return MLA_OK;
}

// Fixed device scratch of mla_decode_noalloc: the split partials of a decode
// call live here instead of in a caller's workspace.  Each device the library
// runs on holds one copy until the process ends.  Host code never passes the
// array's name to a kernel (in host code it is only a stand-in for the
// symbol): its device address is taken once per device with
// hipGetSymbolAddress and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = 96u << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];
void* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of this device's scratch (the current device's), looked up
// on its first use and kept.
mla_status noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_fail(g_scratch_err[dev], "hipGetSymbolAddress(scratch)");
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}

mla_status decode_common(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat, const int32_t* seq_lens,
                         const int32_t* seq_lens_host, int32_t batch, void* out_latent, float* lse, void* workspace,
                         size_t ws_bytes, void* stream, bool fixed_scratch, const void* w_uv = nullptr,
                         float* out = nullptr, int phase = 0);

// Which launches of mla_decode_proj a call enqueues: both, the split attention
// alone (mla_decode_split_kv), or the merge with the output absorption alone
// (mla_merge_out_proj).
constexpr int kPhaseBoth = 0, kPhaseAttention = 1, kPhaseMerge = 2;

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* mla_last_error(void) { return g_err.c_str(); }

}  // extern "C"

namespace {

// Checks and kernel parameters of the RoPE channel (mla_rope_apply and the
// rotation half of mla_rope_absorb_q).
mla_status rope_params(const mla_dims* dims, const mla_paged_cache* cache, const void* q_rope, const int32_t* q_pos,
                       int64_t n_q, void* q_lat, const void* kv_latent, const void* k_rope, const int32_t* kv_seq,
                       const int32_t* kv_pos, int64_t n_kv, mla::RopeParams* out) {
  if (n_q < 0 || n_kv < 0) return fail(MLA_ERR_INVALID_ARG, "n_q and n_kv must be >= 0");
  if (n_q > 0 && (q_rope == nullptr || q_pos == nullptr || q_lat == nullptr))
    return fail(MLA_ERR_INVALID_ARG, "q_rope, q_pos and q_lat are required when n_q > 0");
  if (n_kv > 0) {
    MLA_TRY(check_cache(cache));
    if (kv_latent == nullptr || k_rope == nullptr || kv_seq == nullptr || kv_pos == nullptr)
      return fail(MLA_ERR_INVALID_ARG, "kv_latent, k_rope, kv_seq and kv_pos are required when n_kv > 0");
  }
  if (n_q * dims->n_heads + n_kv > (static_cast<int64_t>(UINT32_MAX) - 3) * 4)
    return fail(MLA_ERR_UNSUPPORTED, "too many rows for one launch");
  mla::RopeParams p{};
  p.n_heads = dims->n_heads;
  p.d_latent = dims->d_latent;
  p.d_rope = dims->d_rope;
  p.dtype = dims->dtype;
  p.work_dtype = dims->work_dtype;
  p.q_rope = q_rope; p.q_pos = q_pos; p.n_q = n_q; p.q_lat = q_lat;
  p.kv_latent = kv_latent; p.k_rope = k_rope; p.kv_seq = kv_seq; p.kv_pos = kv_pos; p.n_kv = n_kv;
  if (n_kv > 0) {
    p.cache = cache->data; p.num_pages = cache->num_pages; p.block_table = cache->block_table;
    p.num_seqs = cache->num_seqs; p.max_pages = cache->max_pages_per_seq;
  }
  p.q_vec = dims->d_rope % 8 == 0 && reinterpret_cast<uintptr_t>(q_rope) % 16 == 0 &&
            reinterpret_cast<uintptr_t>(q_lat) % 16 == 0;
  for (int j = 0; j < dims->d_rope / 2; ++j) p.theta[j] = std::pow(dims->rope_base, -2.0 * j / dims->d_rope);
  p.q_scale = position_ratio(dims);
  *out = p;
  return MLA_OK;
}

// Checks and kernel parameters of the query absorption.
mla_status absorb_params(const mla_dims* dims, const void* q_nope, const void* w_uk, int64_t n_q, void* q_lat,
                         mla::GemmParams* out) {
  if (n_q < 0) return fail(MLA_ERR_INVALID_ARG, "n_q must be >= 0");
  if (n_q > 0 && (q_nope == nullptr || w_uk == nullptr || q_lat == nullptr))
    return fail(MLA_ERR_INVALID_ARG, "q_nope, w_uk and q_lat must be non-NULL");
  if (dims->dtype == MLA_BF16 && (dims->d_head != 128 || dims->d_latent % 128 != 0))
    return fail(MLA_ERR_UNSUPPORTED, "bf16 absorption needs d_head = 128 and d_latent a multiple of 128");
  if (n_q > 65535LL * 512 || n_q * dims->n_heads * dims->d_latent > (1LL << 40))
    return fail(MLA_ERR_UNSUPPORTED, "n_q too large for one launch");
  *out = mla::GemmParams{dims->n_heads, dims->d_head, dims->d_v, dims->d_latent, dims->d_rope, dims->dtype,
                         dims->work_dtype, q_nope, w_uk, q_lat, n_q};
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_rope_apply(const mla_dims* dims, const mla_paged_cache* cache, const void* q_rope,
                          const int32_t* q_pos, int64_t n_q, void* q_lat, const void* kv_latent,
                          const void* k_rope, const int32_t* kv_seq, const int32_t* kv_pos, int64_t n_kv,
                          void* stream) {
  g_err.clear();
  MLA_TRY(check_dims(dims));
  mla::RopeParams p{};
  MLA_TRY(rope_params(dims, cache, q_rope, q_pos, n_q, q_lat, kv_latent, k_rope, kv_seq, kv_pos, n_kv, &p));
  if (n_kv > 0 && debug_validate())
    MLA_TRY(device_check(cache, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, kv_seq, kv_pos, n_kv, stream));
  const hipError_t e = mla::launch_rope(p, as_stream(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "rope launch");
}

mla_status mla_rope_absorb_q(const mla_dims* dims, const mla_paged_cache* cache, const void* q_nope,
                             const void* w_uk, const void* q_rope, const int32_t* q_pos, int64_t n_q, void* q_lat,
                             const void* kv_latent, const void* k_rope, const int32_t* kv_seq,
                             const int32_t* kv_pos, int64_t n_kv, void* stream) {
  g_err.clear();
  MLA_TRY(check_dims(dims));
  mla::RopeParams r{};
  MLA_TRY(rope_params(dims, cache, q_rope, q_pos, n_q, q_lat, kv_latent, k_rope, kv_seq, kv_pos, n_kv, &r));
  mla::GemmParams g{};
  MLA_TRY(absorb_params(dims, q_nope, w_uk, n_q, q_lat, &g));
  if (n_q == 0 && n_kv == 0) return MLA_OK;
  if (n_kv > 0 && debug_validate())
    MLA_TRY(device_check(cache, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, kv_seq, kv_pos, n_kv, stream));
  const hipError_t e = mla::launch_rope_absorb(g, r, as_stream(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "rope + absorb launch");
}

mla_status mla_absorb_q(const mla_dims* dims, const void* q_nope, const void* w_uk, int64_t n_q, void* q_lat,
                        void* stream) {
  g_err.clear();
  MLA_TRY(check_dims(dims));
  mla::GemmParams p{};
  MLA_TRY(absorb_params(dims, q_nope, w_uk, n_q, q_lat, &p));
  if (n_q == 0) return MLA_OK;
  const hipError_t e = mla::launch_absorb(p, as_stream(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "absorb launch");
}

mla_status mla_out_proj(const mla_dims* dims, const void* out_latent, const void* w_uv, int64_t n, void* out,
                        void* stream) {
  g_err.clear();
  MLA_TRY(check_dims(dims));
  if (n < 0) return fail(MLA_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return MLA_OK;
  if (out_latent == nullptr || w_uv == nullptr || out == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "out_latent, w_uv and out must be non-NULL");
  if (dims->dtype == MLA_BF16 && (dims->d_latent % 32 != 0 || dims->d_latent > 512 || dims->d_v % 64 != 0))
    return fail(MLA_ERR_UNSUPPORTED, "bf16 output projection needs d_latent a multiple of 32 up to 512 and d_v a "
                                     "multiple of 64");
  if (n > (1LL << 31) / dims->n_heads) return fail(MLA_ERR_UNSUPPORTED, "n too large for one launch");
  if (dims->dtype == MLA_F32 && n * dims->n_heads * static_cast<int64_t>(dims->d_v) / 4 >= (1LL << 31))
    return fail(MLA_ERR_UNSUPPORTED, "n too large for one float32 launch");
  mla::GemmParams p{dims->n_heads, dims->d_head, dims->d_v, dims->d_latent, dims->d_rope, dims->dtype,
                    dims->work_dtype, out_latent, w_uv, out, n};
  const hipError_t e = mla::launch_out_proj(p, as_stream(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "out_proj launch");
}

mla_status mla_decode_plan(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host, int32_t* split_pages,
                           int64_t* n_items) {
  g_err.clear();
  MLA_TRY(check_dims(dims));
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 0");
  if (batch > 0 && seq_lens_host == nullptr) return fail(MLA_ERR_INVALID_ARG, "seq_lens_host is NULL");
  const Plan p = make_plan(dims, batch, seq_lens_host);
  if (split_pages) *split_pages = p.split_pages;
  if (n_items) *n_items = p.n_items;
  return MLA_OK;
}

size_t mla_decode_workspace_size(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host) {
  if (check_dims(dims) != MLA_OK || batch <= 0 || seq_lens_host == nullptr) return 0;
  return workspace_bytes(dims, make_plan(dims, batch, seq_lens_host));
}

mla_status mla_decode(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat, const int32_t* seq_lens,
                      const int32_t* seq_lens_host, int32_t batch, void* out_latent, float* lse, void* workspace,
                      size_t ws_bytes, void* stream) {
  g_err.clear();
  return decode_common(dims, cache, q_lat, seq_lens, seq_lens_host, batch, out_latent, lse, workspace, ws_bytes,
                       stream, false);
}

size_t mla_decode_proj_workspace_size(const mla_dims* dims, int32_t batch, const int32_t* seq_lens_host) {
  if (check_dims(dims) != MLA_OK || batch <= 0 || seq_lens_host == nullptr) return 0;
  return proj_workspace_bytes(dims, make_plan(dims, batch, seq_lens_host), batch);
}

mla_status mla_decode_proj(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                           const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch, const void* w_uv,
                           void* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (w_uv == nullptr || out == nullptr) return fail(MLA_ERR_INVALID_ARG, "w_uv and out must be non-NULL");
  return decode_common(dims, cache, q_lat, seq_lens, seq_lens_host, batch, nullptr, lse, workspace, ws_bytes,
                       stream, false, w_uv, static_cast<float*>(out));
}

mla_status mla_decode_split_kv(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                               const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch, void* workspace,
                               size_t ws_bytes, void* stream) {
  g_err.clear();
  return decode_common(dims, cache, q_lat, seq_lens, seq_lens_host, batch, nullptr, nullptr, workspace, ws_bytes,
                       stream, false, nullptr, nullptr, kPhaseAttention);
}

mla_status mla_merge_out_proj(const mla_dims* dims, const int32_t* seq_lens, const int32_t* seq_lens_host,
                              int32_t batch, const void* w_uv, void* out, float* lse, const void* workspace,
                              size_t ws_bytes, void* stream) {
  g_err.clear();
  if (w_uv == nullptr || out == nullptr) return fail(MLA_ERR_INVALID_ARG, "w_uv and out must be non-NULL");
  return decode_common(dims, nullptr, nullptr, seq_lens, seq_lens_host, batch, nullptr, lse,
                       const_cast<void*>(workspace), ws_bytes, stream, false, w_uv, static_cast<float*>(out),
                       kPhaseMerge);
}

mla_status mla_decode_noalloc(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                              const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch, void* out_latent,
                              float* lse, void* stream) {
  g_err.clear();
  void* scratch_ptr = nullptr;
  MLA_TRY(noalloc_scratch(&scratch_ptr));
  return decode_common(dims, cache, q_lat, seq_lens, seq_lens_host, batch, out_latent, lse, scratch_ptr,
                       kNoAllocScratchBytes, stream, true);
}

}  // extern "C"

namespace {

mla_status decode_common(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat, const int32_t* seq_lens,
                         const int32_t* seq_lens_host, int32_t batch, void* out_latent, float* lse, void* workspace,
                         size_t ws_bytes, void* stream, bool fixed_scratch, const void* w_uv, float* out,
                         int phase) {
  const bool attend = phase != kPhaseMerge;  // this call launches the attention
  MLA_TRY(check_dims(dims));
  MLA_TRY(check_attn_shape(dims));
  if (attend) MLA_TRY(check_cache(cache));
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 0");
  if (batch == 0) return MLA_OK;
  if (attend && batch > cache->num_seqs)
    return fail(MLA_ERR_INVALID_ARG, "batch (%d) exceeds the block table's rows (%d)", batch, cache->num_seqs);
  // mla_decode_proj, or one of its two launches: every work item leaves a partial
  const bool fused = w_uv != nullptr || out != nullptr || phase != kPhaseBoth;
  if ((attend && q_lat == nullptr) || seq_lens == nullptr || seq_lens_host == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "q_lat, seq_lens and seq_lens_host must be non-NULL");
  if (!fused && out_latent == nullptr) return fail(MLA_ERR_INVALID_ARG, "out_latent must be non-NULL");
  if (fused && phase != kPhaseAttention && (w_uv == nullptr || out == nullptr))
    return fail(MLA_ERR_INVALID_ARG, "w_uv and out must be non-NULL");
  if (fused && dims->d_v != 128) return fail(MLA_ERR_UNSUPPORTED, "mla_decode_proj needs d_v = 128");
  if (phase != kPhaseBoth && dims->dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_split_kv and mla_merge_out_proj take bf16 caches only");
  for (int b = 0; b < batch; ++b) {
    if (seq_lens_host[b] < 0 ||
        (attend &&
         static_cast<int64_t>(seq_lens_host[b]) > static_cast<int64_t>(cache->max_pages_per_seq) * mla::kPage))
      return fail(MLA_ERR_INVALID_ARG, "seq_lens_host[%d] = %d is negative or beyond the block table", b,
                  seq_lens_host[b]);
    if (attend && seq_lens_host[b] > 0 && cache->num_pages == 0)
      return fail(MLA_ERR_INVALID_ARG, "sequence %d has tokens but the cache has no pages", b);
  }
  if (attend && debug_validate())
    MLA_TRY(device_check(cache, batch, seq_lens, seq_lens_host, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                         stream));
  mla::AttnParams p{};
  p.n_heads = dims->n_heads; p.d_latent = dims->d_latent; p.d_rope = dims->d_rope;
  p.f32w = dims->work_dtype == MLA_F32;
  p.scale = dims->softmax_scale;
  p.scale_log2 = static_cast<float>(dims->softmax_scale * 1.4426950408889634);
  if (attend) {
    p.q_lat = q_lat; p.cache = cache->data; p.num_pages = cache->num_pages; p.block_table = cache->block_table;
    p.num_seqs = cache->num_seqs; p.max_pages = cache->max_pages_per_seq;
  }
  p.seq_lens = seq_lens; p.batch = batch; p.out_latent = out_latent; p.lse = lse;
  hipStream_t s = as_stream(stream);
  const Plan plan = make_plan(dims, batch, seq_lens_host);
  const size_t need = fused ? proj_workspace_bytes(dims, plan, batch) : workspace_bytes(dims, plan);
  if (fused && need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(MLA_ERR_WORKSPACE, "decode_proj needs %zu bytes of workspace, got %zu", need,
                workspace ? ws_bytes : 0);
  if (dims->dtype == MLA_F32) {
    // float32 path: obar goes through the workspace to the output absorption
    if (fused) p.out_latent = workspace;
    hipError_t e = mla::launch_decode_f32(p, s);
    if (e != hipSuccess || !fused) return e == hipSuccess ? MLA_OK : hip_fail(e, "decode launch");
    const mla::GemmParams g{dims->n_heads, dims->d_head, dims->d_v, dims->d_latent, dims->d_rope, dims->dtype,
                            dims->work_dtype, workspace, w_uv, out, batch};
    e = mla::launch_out_proj(g, s);
    return e == hipSuccess ? MLA_OK : hip_fail(e, "out_proj launch");
  }
  if (fixed_scratch && need > ws_bytes)
    return fail(MLA_ERR_WORKSPACE,
                "mla_decode_noalloc: this batch needs %zu bytes of split partials, more than its fixed scratch of %zu "
                "bytes; use mla_decode with a workspace", need, ws_bytes);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(MLA_ERR_WORKSPACE, "decode needs %zu bytes of workspace, got %zu", need, workspace ? ws_bytes : 0);
  if (plan.n_items > (1LL << 31) - 1) return fail(MLA_ERR_UNSUPPORTED, "too many work items");
  p.split_pages = plan.split_pages;
  p.n_full = plan.n_full;
  p.n_items = plan.n_items;
  p.n_head_chunks = 1;
  p.all_partials = fused ? 1 : 0;
  if (need > 0) {
    p.ws_o = static_cast<float*>(workspace);
    p.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + partial_bytes(dims, plan));
    if (half_partials(dims)) {
      p.half_partials = 1;
      p.ws_exp = reinterpret_cast<int32_t*>(
          static_cast<char*>(workspace) +
          align_ws(static_cast<size_t>(plan.n_items) * dims->n_heads * dims->d_latent * 2));
    }
  }
  hipError_t e = hipSuccess;
  if (attend) {
    e = mla::launch_decode_bf16(p, s);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  }
  if (phase == kPhaseAttention) return MLA_OK;
  if (fused) {
    const mla::GemmParams g{dims->n_heads, dims->d_head, dims->d_v, dims->d_latent, dims->d_rope, dims->dtype,
                            dims->work_dtype, nullptr, w_uv, out, batch};
    e = mla::launch_merge_proj(g, p, s);
    return e == hipSuccess ? MLA_OK : hip_fail(e, "merge + output absorption launch");
  }
  if (plan.needs_merge) {
    e = mla::launch_merge(p, s);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

// ---- per-head position keys (rows [c | R k^R_0 | ... | R k^R_{H-1}])

namespace {

mla_status check_per_head_shape(const mla_dims* d) {
  if (d->dtype != MLA_BF16 || d->n_heads != 16 || d->d_latent != 256 || d->d_rope != 32)
    return fail(MLA_ERR_UNSUPPORTED,
                "per-head position keys need bf16, 16 heads, d_latent 256 and d_rope 32 (got %d heads, %d, %d)",
                d->n_heads, d->d_latent, d->d_rope);
  return MLA_OK;
}

}  // namespace

mla_status mla_cache_write_per_head(const mla_dims* dims, const mla_paged_cache* cache, const void* kv_latent,
                                    const void* k_rope, const int32_t* kv_seq, const int32_t* kv_pos, int64_t n_kv,
                                    void* stream) {
  g_err.clear();
  MLA_TRY(check_dims(dims));
  MLA_TRY(check_per_head_shape(dims));
  if (n_kv < 0) return fail(MLA_ERR_INVALID_ARG, "n_kv must be >= 0");
  if (n_kv == 0) return MLA_OK;
  MLA_TRY(check_cache(cache));
  if (kv_latent == nullptr || k_rope == nullptr || kv_seq == nullptr || kv_pos == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "kv_latent, k_rope, kv_seq and kv_pos must be non-NULL");
  if (n_kv > (static_cast<int64_t>(UINT32_MAX) - 3) * 4) return fail(MLA_ERR_UNSUPPORTED, "too many rows for one launch");
  if (debug_validate())
    MLA_TRY(device_check(cache, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, kv_seq, kv_pos, n_kv, stream));
  mla::RopeParams p{};
  p.n_heads = dims->n_heads; p.d_latent = dims->d_latent; p.d_rope = dims->d_rope;
  p.dtype = dims->dtype; p.work_dtype = dims->work_dtype;
  p.kv_latent = kv_latent; p.k_rope = k_rope; p.kv_seq = kv_seq; p.kv_pos = kv_pos; p.n_kv = n_kv;
  p.cache = cache->data; p.num_pages = cache->num_pages; p.block_table = cache->block_table;
  p.num_seqs = cache->num_seqs; p.max_pages = cache->max_pages_per_seq;
  p.q_scale = 1.0;
  for (int j = 0; j < dims->d_rope / 2; ++j) p.theta[j] = std::pow(dims->rope_base, -2.0 * j / dims->d_rope);
  const hipError_t e = mla::launch_perhead_cache_write(p, as_stream(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "per-head cache write launch");
}

namespace {

// mla_decode_per_head, or with w_uv and out (mla_decode_per_head_proj) the
// fused merge and output absorption in place of the merge
mla_status per_head_common(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                           const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch, void* out_latent,
                           float* lse, void* workspace, size_t ws_bytes, void* stream, const void* w_uv, float* out) {
  const bool fused = w_uv != nullptr || out != nullptr;
  MLA_TRY(check_dims(dims));
  MLA_TRY(check_per_head_shape(dims));
  MLA_TRY(check_cache(cache));
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 0");
  if (batch == 0) return MLA_OK;
  if (batch > cache->num_seqs)
    return fail(MLA_ERR_INVALID_ARG, "batch (%d) exceeds the block table's rows (%d)", batch, cache->num_seqs);
  if (q_lat == nullptr || seq_lens == nullptr || seq_lens_host == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "q_lat, seq_lens and seq_lens_host must be non-NULL");
  if (!fused && out_latent == nullptr) return fail(MLA_ERR_INVALID_ARG, "out_latent must be non-NULL");
  if (fused && (w_uv == nullptr || out == nullptr)) return fail(MLA_ERR_INVALID_ARG, "w_uv and out must be non-NULL");
  if (fused && dims->d_v != 128) return fail(MLA_ERR_UNSUPPORTED, "the fused output absorption needs d_v = 128");
  for (int b = 0; b < batch; ++b) {
    if (seq_lens_host[b] < 0 ||
        static_cast<int64_t>(seq_lens_host[b]) > static_cast<int64_t>(cache->max_pages_per_seq) * mla::kPage)
      return fail(MLA_ERR_INVALID_ARG, "seq_lens_host[%d] = %d is negative or beyond the block table", b,
                  seq_lens_host[b]);
    if (seq_lens_host[b] > 0 && cache->num_pages == 0)
      return fail(MLA_ERR_INVALID_ARG, "sequence %d has tokens but the cache has no pages", b);
  }
  if (debug_validate())
    MLA_TRY(device_check(cache, batch, seq_lens, seq_lens_host, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                         stream));
  const Plan plan = make_plan(dims, batch, seq_lens_host);
  const size_t need = fused ? proj_workspace_bytes(dims, plan, batch) : workspace_bytes(dims, plan);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(MLA_ERR_WORKSPACE, "decode needs %zu bytes of workspace, got %zu", need, workspace ? ws_bytes : 0);
  if (plan.n_items > (1LL << 31) - 1) return fail(MLA_ERR_UNSUPPORTED, "too many work items");
  mla::AttnParams p{};
  p.n_heads = dims->n_heads; p.d_latent = dims->d_latent; p.d_rope = dims->d_rope;
  p.f32w = dims->work_dtype == MLA_F32;
  p.scale = dims->softmax_scale;
  p.scale_log2 = static_cast<float>(dims->softmax_scale * 1.4426950408889634);
  p.q_lat = q_lat; p.cache = cache->data; p.num_pages = cache->num_pages; p.block_table = cache->block_table;
  p.num_seqs = cache->num_seqs; p.max_pages = cache->max_pages_per_seq;
  p.seq_lens = seq_lens; p.batch = batch; p.out_latent = out_latent; p.lse = lse;
  p.split_pages = plan.split_pages; p.n_full = plan.n_full; p.n_items = plan.n_items; p.n_head_chunks = 1;
  p.all_partials = fused ? 1 : 0;
  if (need > 0) {
    p.ws_o = static_cast<float*>(workspace);
    p.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + partial_bytes(dims, plan));
  }
  const hipStream_t s = as_stream(stream);
  hipError_t e = mla::launch_perhead_decode(p, s);
  if (e != hipSuccess) return hip_fail(e, "per-head decode launch");
  if (fused) {
    const mla::GemmParams g{dims->n_heads, dims->d_head, dims->d_v, dims->d_latent, dims->d_rope, dims->dtype,
                            dims->work_dtype, nullptr, w_uv, out, batch};
    e = mla::launch_merge_proj(g, p, s);
    return e == hipSuccess ? MLA_OK : hip_fail(e, "merge + output absorption launch");
  }
  if (plan.needs_merge) {
    e = mla::launch_merge(p, s);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return MLA_OK;
}

}  // namespace

mla_status mla_decode_per_head(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                               const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch, void* out_latent,
                               float* lse, void* workspace, size_t ws_bytes, void* stream) {
  g_err.clear();
  return per_head_common(dims, cache, q_lat, seq_lens, seq_lens_host, batch, out_latent, lse, workspace, ws_bytes,
                         stream, nullptr, nullptr);
}

mla_status mla_decode_per_head_proj(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat,
                                    const int32_t* seq_lens, const int32_t* seq_lens_host, int32_t batch,
                                    const void* w_uv, void* out, float* lse, void* workspace, size_t ws_bytes,
                                    void* stream) {
  g_err.clear();
  if (w_uv == nullptr || out == nullptr) return fail(MLA_ERR_INVALID_ARG, "w_uv and out must be non-NULL");
  return per_head_common(dims, cache, q_lat, seq_lens, seq_lens_host, batch, nullptr, lse, workspace, ws_bytes,
                         stream, w_uv, static_cast<float*>(out));
}

mla_status mla_prefill(const mla_dims* dims, const mla_paged_cache* cache, const void* q_lat, const int32_t* cu_q,
                       const int32_t* q_start_pos, const int32_t* cu_q_host, const int32_t* q_start_pos_host,
                       int32_t batch, void* out_latent, float* lse, void* stream) {
  g_err.clear();
  MLA_TRY(check_dims(dims));
  MLA_TRY(check_attn_shape(dims));
  MLA_TRY(check_cache(cache));
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 0");
  if (batch == 0) return MLA_OK;
  if (batch > cache->num_seqs)
    return fail(MLA_ERR_INVALID_ARG, "batch (%d) exceeds the block table's rows (%d)", batch, cache->num_seqs);
  if (q_lat == nullptr || cu_q == nullptr || q_start_pos == nullptr || cu_q_host == nullptr ||
      q_start_pos_host == nullptr || out_latent == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "q_lat, cu_q, q_start_pos, their host copies and out_latent must be non-NULL");
  if (cu_q_host[0] != 0) return fail(MLA_ERR_INVALID_ARG, "cu_q[0] must be 0");
  const int rows = 128;  // (query, head) rows per bf16 workgroup
  int64_t n_blocks = 0;
  for (int b = 0; b < batch; ++b) {
    const int nq = cu_q_host[b + 1] - cu_q_host[b];
    if (nq < 0) return fail(MLA_ERR_INVALID_ARG, "cu_q must be non-decreasing (at %d)", b);
    if (q_start_pos_host[b] < 0) return fail(MLA_ERR_INVALID_ARG, "q_start_pos[%d] is negative", b);
    const int64_t last = static_cast<int64_t>(q_start_pos_host[b]) + nq;
    if (last > 0 && cache->num_pages == 0)
      return fail(MLA_ERR_INVALID_ARG, "sequence %d has tokens but the cache has no pages", b);
    if (last > static_cast<int64_t>(cache->max_pages_per_seq) * mla::kPage)
      return fail(MLA_ERR_INVALID_ARG, "sequence %d reaches position %lld beyond its block table", b,
                  static_cast<long long>(last - 1));
    if (nq > 0 && static_cast<int64_t>(nq) * dims->n_heads > (1LL << 31) - 1)
      return fail(MLA_ERR_UNSUPPORTED, "too many query rows in sequence %d", b);
    n_blocks += dims->dtype == MLA_BF16 ? (static_cast<int64_t>(nq) * dims->n_heads + rows - 1) / rows
                                        : static_cast<int64_t>(nq) * dims->n_heads;
  }
  if (n_blocks == 0) return MLA_OK;
  if (n_blocks > (1LL << 31) - 1) return fail(MLA_ERR_UNSUPPORTED, "too many workgroups");
  if (debug_validate())
    MLA_TRY(device_check(cache, batch, nullptr, nullptr, cu_q, q_start_pos, cu_q_host, q_start_pos_host, nullptr,
                         nullptr, 0, stream));
  mla::AttnParams p{};
  p.n_heads = dims->n_heads; p.d_latent = dims->d_latent; p.d_rope = dims->d_rope;
  p.f32w = dims->work_dtype == MLA_F32;
  p.scale = dims->softmax_scale;
  p.scale_log2 = static_cast<float>(dims->softmax_scale * 1.4426950408889634);
  p.q_lat = q_lat; p.cache = cache->data; p.num_pages = cache->num_pages; p.block_table = cache->block_table;
  p.num_seqs = cache->num_seqs; p.max_pages = cache->max_pages_per_seq;
  p.batch = batch; p.cu_q = cu_q; p.q_start = q_start_pos; p.n_blocks = n_blocks;
  p.out_latent = out_latent; p.lse = lse;
  const hipError_t e = dims->dtype == MLA_BF16 ? mla::launch_prefill_bf16(p, as_stream(stream))
                                               : mla::launch_prefill_f32(p, as_stream(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "prefill launch");
}

// ---------------------------------------------------- materialised prefill

namespace {

struct MhaPlan {
  int64_t n_keys = 0, n_key_tiles = 0, n_q_blocks = 0;
};

mla_status plan_mha(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch, const int32_t* cu_q_host,
                    const int32_t* q_start_pos_host, MhaPlan* plan) {
  MLA_TRY(check_dims(dims));
  if (dims->dtype != MLA_BF16 || dims->work_dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "the materialised prefill is bf16 only (dtype and work_dtype)");
  if (dims->d_head != 128 || dims->d_v != 128)
    return fail(MLA_ERR_UNSUPPORTED, "the materialised prefill needs d_head = d_v = 128 (got %d, %d)", dims->d_head,
                dims->d_v);
  const bool dsv2 = dims->n_heads == 128 && dims->d_latent == 512 && dims->d_rope == 64;
  const bool tiny = dims->n_heads == 16 && dims->d_latent == 256 && dims->d_rope == 32;
  if (!dsv2 && !tiny)
    return fail(MLA_ERR_UNSUPPORTED, "materialised prefill supports (n_heads, d_latent, d_rope) = (128, 512, 64) or "
                "(16, 256, 32); got (%d, %d, %d)", dims->n_heads, dims->d_latent, dims->d_rope);
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 0");
  if (batch > 0 && (cu_q_host == nullptr || q_start_pos_host == nullptr))
    return fail(MLA_ERR_INVALID_ARG, "cu_q_host and q_start_pos_host must be non-NULL");
  if (batch > 0 && cu_q_host[0] != 0) return fail(MLA_ERR_INVALID_ARG, "cu_q[0] must be 0");
  if (cache != nullptr && batch > cache->num_seqs)
    return fail(MLA_ERR_INVALID_ARG, "batch (%d) exceeds the block table's rows (%d)", batch, cache->num_seqs);
  MhaPlan pl;
  for (int b = 0; b < batch; ++b) {
    const int nq = cu_q_host[b + 1] - cu_q_host[b];
    if (nq < 0) return fail(MLA_ERR_INVALID_ARG, "cu_q must be non-decreasing (at %d)", b);
    if (q_start_pos_host[b] < 0) return fail(MLA_ERR_INVALID_ARG, "q_start_pos[%d] is negative", b);
    const int64_t T = static_cast<int64_t>(q_start_pos_host[b]) + nq;
    if (cache != nullptr && T > static_cast<int64_t>(cache->max_pages_per_seq) * mla::kPage)
      return fail(MLA_ERR_INVALID_ARG, "sequence %d reaches position %lld beyond its block table", b,
                  static_cast<long long>(T - 1));
    if (cache != nullptr && T > 0 && cache->num_pages == 0)
      return fail(MLA_ERR_INVALID_ARG, "sequence %d has tokens but the cache has no pages", b);
    pl.n_keys += (T + 127) / 128 * 128;  // each sequence's keys take a range padded to 128
    pl.n_key_tiles += (T + 255) / 256;
    pl.n_q_blocks += (nq + 127) / 128 * dims->n_heads;
  }
  if (pl.n_key_tiles * dims->n_heads > (1LL << 31) - 1 || pl.n_q_blocks > (1LL << 31) - 1)
    return fail(MLA_ERR_UNSUPPORTED, "too many workgroups for one launch");
  // the transposed values are addressed with 32-bit byte offsets within a head: 127 rows of n_keys
  // plus one sequence's range
  if (pl.n_keys > (1LL << 24) - 128)
    return fail(MLA_ERR_UNSUPPORTED, "materialised prefill of %lld padded key positions (at most %lld)",
                static_cast<long long>(pl.n_keys), (1LL << 24) - 128);
  *plan = pl;
  return MLA_OK;
}

size_t mha_ws_half(const mla_dims* dims, int64_t n_keys) {
  const size_t half = static_cast<size_t>(dims->n_heads) * static_cast<size_t>(n_keys) * 128 * sizeof(uint16_t);
  return (half + kWsAlign - 1) / kWsAlign * kWsAlign;
}

}  // namespace

size_t mla_prefill_mha_workspace_size(const mla_dims* dims, int32_t batch, const int32_t* cu_q_host,
                                      const int32_t* q_start_pos_host) {
  g_err.clear();
  MhaPlan pl;
  if (plan_mha(dims, nullptr, batch, cu_q_host, q_start_pos_host, &pl) != MLA_OK) return 0;
  return 2 * mha_ws_half(dims, pl.n_keys);
}

mla_status mla_prefill_mha(const mla_dims* dims, const mla_paged_cache* cache, const void* q_nope, const void* q_lat,
                           const void* w_uk, const void* w_uv, const int32_t* cu_q, const int32_t* q_start_pos,
                           const int32_t* cu_q_host, const int32_t* q_start_pos_host, int32_t batch, float* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  MLA_TRY(check_dims(dims));
  MLA_TRY(check_cache(cache));
  MhaPlan pl;
  MLA_TRY(plan_mha(dims, cache, batch, cu_q_host, q_start_pos_host, &pl));
  if (pl.n_keys == 0) return MLA_OK;
  if (q_nope == nullptr || q_lat == nullptr || w_uk == nullptr || w_uv == nullptr || cu_q == nullptr ||
      q_start_pos == nullptr || out == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "q_nope, q_lat, w_uk, w_uv, cu_q, q_start_pos and out must be non-NULL");
  const size_t half = mha_ws_half(dims, pl.n_keys);
  if (workspace == nullptr || workspace_bytes < 2 * half)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, 2 * half);
  if (debug_validate())
    MLA_TRY(device_check(cache, batch, nullptr, nullptr, cu_q, q_start_pos, cu_q_host, q_start_pos_host, nullptr,
                         nullptr, 0, stream));
  mla::MhaParams p{};
  p.n_heads = dims->n_heads; p.d_latent = dims->d_latent; p.d_rope = dims->d_rope;
  p.scale_log2 = static_cast<float>(dims->softmax_scale * 1.4426950408889634);
  p.cache = cache->data; p.num_pages = cache->num_pages; p.block_table = cache->block_table;
  p.num_seqs = cache->num_seqs; p.max_pages = cache->max_pages_per_seq;
  p.cu_q = cu_q; p.q_start = q_start_pos; p.batch = batch;
  p.q_nope = q_nope; p.q_lat = q_lat; p.w_uk = w_uk; p.w_uv = w_uv;
  p.ws_k = static_cast<uint16_t*>(workspace);
  p.ws_v = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + half);
  p.n_keys = pl.n_keys; p.n_key_tiles = pl.n_key_tiles; p.n_q_blocks = pl.n_q_blocks;
  p.out = out; p.lse = lse;
  const hipError_t e = mla::launch_mha_prefill(p, as_stream(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "materialised prefill launch");
}

}  // extern "C"

namespace {

// ---- front of the layer ---------------------------------------------------

// Splits of K for an [m x n x k] projection: the first count (a divisor of
// k / 32, at most k / 256) that gives two workgroups per CU, else the largest.
// Split-K factor of a projection: the smallest s (a divisor of k / 32, at
// least eight slices a split) that gives two workgroups a CU; when that count
// leaves the CUs unevenly loaded and a larger s still fits three a CU (all
// resident at once) with an even count, that s, so no CU streams a third
// more weights than the rest.
int front_splits(int64_t m, int64_t n, int k) {
  const int64_t tiles = ((m + 63) / 64) * ((n + 127) / 128);
  int best = 1, fallback = 0;
  for (int s = 1; s <= k / 256 && s <= 64; ++s) {
    if (k % (32 * s) != 0) continue;
    const int64_t wgs = tiles * s;
    if (fallback == 0) best = s;
    if (wgs < 2 * kPlanCUs) continue;
    if (wgs > 3 * kPlanCUs) break;
    if (wgs % kPlanCUs == 0) return s;
    if (fallback == 0) fallback = s;
  }
  return fallback != 0 ? fallback : best;
}

size_t front_part_bytes(int64_t m, int64_t n, int k) {
  return static_cast<size_t>(front_splits(m, n, k)) * static_cast<size_t>(m) * static_cast<size_t>(n) * 4;
}

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

mla_status check_front(const mla_dims* d, int64_t n, int32_t d_model, int32_t d_qlat, bool need_q) {
  MLA_TRY(check_dims(d));
  if (d->dtype != MLA_BF16 || d->work_dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "the front projections are bf16 only");
  if (n < 0) return fail(MLA_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 65535LL * 64) return fail(MLA_ERR_UNSUPPORTED, "more than %lld tokens in one call", 65535LL * 64);
  if (d_model <= 0 || d_model % 32 != 0)
    return fail(MLA_ERR_INVALID_ARG, "d_model must be a positive multiple of 32 (got %d)", d_model);
  if ((need_q && d_qlat <= 0) || d_qlat < 0 || d_qlat % 32 != 0)
    return fail(MLA_ERR_INVALID_ARG, "d_qlat must be a positive multiple of 32 (got %d)", d_qlat);
  if (d->d_latent % 16 != 0 || (d->n_heads * d->d_head) % 16 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "d_latent and n_heads * d_head must be multiples of 16");
  const int64_t widest = static_cast<int64_t>(d->n_heads) * (d->d_latent + d->d_rope);
  if (widest > (1LL << 30) || static_cast<int64_t>(d_model) * (d->d_latent + d->d_rope) * 2 > 0xffffffffLL ||
      static_cast<int64_t>(d_qlat) * widest * 2 > 0xffffffffLL)
    return fail(MLA_ERR_UNSUPPORTED, "a weight over 4 GiB");
  return MLA_OK;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

size_t front_ws(const mla_dims* d, int64_t n, int32_t d_model, int32_t d_qlat) {
  const int64_t kv_n = d->d_latent + d->d_rope;
  size_t part = front_part_bytes(n, kv_n, d_model);
  if (d_qlat > 0) {
    part = std::max(part, front_part_bytes(n, d_qlat, d_model));
    part = std::max(part, front_part_bytes(n, static_cast<int64_t>(d->n_heads) * (d->d_head + d->d_rope), d_qlat));
    part = std::max(part, front_part_bytes(n, static_cast<int64_t>(d->n_heads) * (d->d_latent + d->d_rope), d_qlat));
  }
  return align_up(part) + align_up(static_cast<size_t>(n) * static_cast<size_t>(d_qlat) * 2);
}

void set_theta(const mla_dims* d, double* theta) {
  for (int j = 0; j < d->d_rope / 2; ++j) theta[j] = std::pow(d->rope_base, -2.0 * j / d->d_rope);
}

// One projection: Y = X [m, k] W^T with W rows [0, n1) from w1 and [n1, n) from w2,
// then the reduce that writes its destination.
mla_status front_project(const mla::bf16_t* x, int64_t ldx, int64_t m, int k, const void* w1, const void* w2, int64_t n,
                         int64_t n1, float* part, mla::FrontReduceParams rp, int mode, hipStream_t st) {
  mla::GemmNtParams g{};
  g.x = x; g.ldx = ldx;
  g.w1 = static_cast<const mla::bf16_t*>(w1); g.w2 = static_cast<const mla::bf16_t*>(w2 != nullptr ? w2 : w1);
  g.m = static_cast<int>(m); g.n = static_cast<int>(n); g.n1 = static_cast<int>(n1); g.k = k;
  const int splits = front_splits(m, n, k);
  g.k_split = k / splits;
  g.part = part;
  hipError_t e = mla::launch_gemm_nt(g, splits, st);
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  rp.part = part; rp.splits = splits; rp.m = static_cast<int>(m); rp.n = static_cast<int>(n);
  e = mla::launch_front_reduce(rp, mode, st);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "projection reduce launch");
}

}  // namespace

extern "C" {

size_t mla_front_workspace_size(const mla_dims* dims, int64_t n, int32_t d_model, int32_t d_qlat) {
  g_err.clear();
  if (check_front(dims, n, d_model, d_qlat, false) != MLA_OK) return 0;
  return front_ws(dims, n, d_model, d_qlat);
}

mla_status mla_kv_project(const mla_dims* dims, const mla_paged_cache* cache, const void* h, int64_t n,
                          int32_t d_model, const void* w_dkv, const void* w_kr, const int32_t* kv_seq,
                          const int32_t* kv_pos, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  MLA_TRY(check_front(dims, n, d_model, 0, false));
  if (n == 0) return MLA_OK;
  MLA_TRY(check_cache(cache));
  if (h == nullptr || w_dkv == nullptr || w_kr == nullptr || kv_seq == nullptr || kv_pos == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "h, w_dkv, w_kr, kv_seq and kv_pos must be non-NULL");
  if (!aligned16(h) || !aligned16(w_dkv) || !aligned16(w_kr))
    return fail(MLA_ERR_INVALID_ARG, "h and the weights must be 16-byte aligned");
  const size_t need = front_ws(dims, n, d_model, 0);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  mla::FrontReduceParams rp{};
  rp.n_heads = dims->n_heads; rp.d_head = dims->d_head; rp.d_latent = dims->d_latent; rp.d_rope = dims->d_rope;
  rp.cache = cache->data; rp.num_pages = cache->num_pages; rp.block_table = cache->block_table;
  rp.max_pages = cache->max_pages_per_seq; rp.kv_seq = kv_seq; rp.kv_pos = kv_pos;
  set_theta(dims, rp.theta);
  return front_project(static_cast<const mla::bf16_t*>(h), d_model, n, d_model, w_dkv, w_kr,
                       dims->d_latent + dims->d_rope, dims->d_latent, static_cast<float*>(workspace), rp,
                       mla::kFrontKv, as_stream(stream));
}

static mla_status q_project_impl(const mla_dims* dims, const void* h, int64_t n, int32_t d_model, int32_t d_qlat,
                                 const void* w_dq, const void* w_up, const void* w_qr, const int32_t* q_pos,
                                 void* q_nope, void* q_lat, void* workspace, size_t workspace_bytes, void* stream,
                                 bool folded) {
  g_err.clear();
  MLA_TRY(check_front(dims, n, d_model, d_qlat, true));
  if (n == 0) return MLA_OK;
  if (h == nullptr || w_dq == nullptr || w_up == nullptr || w_qr == nullptr || q_pos == nullptr ||
      q_lat == nullptr || (!folded && q_nope == nullptr))
    return fail(MLA_ERR_INVALID_ARG, folded ? "h, w_dq, w_fold, w_qr, q_pos and q_lat must be non-NULL"
                                            : "h, w_dq, w_uq, w_qr, q_pos, q_nope and q_lat must be non-NULL");
  if (!aligned16(h) || !aligned16(w_dq) || !aligned16(w_up) || !aligned16(w_qr))
    return fail(MLA_ERR_INVALID_ARG, "h and the weights must be 16-byte aligned");
  const size_t need = front_ws(dims, n, d_model, d_qlat);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  const size_t part_bytes = need - align_up(static_cast<size_t>(n) * static_cast<size_t>(d_qlat) * 2);
  float* part = static_cast<float*>(workspace);
  mla::bf16_t* cq = reinterpret_cast<mla::bf16_t*>(static_cast<char*>(workspace) + part_bytes);
  const hipStream_t st = as_stream(stream);
  // the query latent c^Q = W_DQ h, kept in bf16
  mla::FrontReduceParams rp{};
  rp.n_heads = dims->n_heads; rp.d_head = dims->d_head; rp.d_latent = dims->d_latent; rp.d_rope = dims->d_rope;
  rp.y = cq; rp.ldy = d_qlat;
  set_theta(dims, rp.theta);
  MLA_TRY(front_project(static_cast<const mla::bf16_t*>(h), d_model, n, d_model, w_dq, nullptr, d_qlat, d_qlat, part, rp,
                        mla::kFrontPlain, st));
  // the content (or folded) and position queries from c^Q
  rp.y = nullptr;
  rp.q_nope = static_cast<mla::bf16_t*>(q_nope); rp.q_lat = static_cast<mla::bf16_t*>(q_lat); rp.q_pos = q_pos;
  rp.q_scale = position_ratio(dims);
  const int64_t w0 = folded ? dims->d_latent : dims->d_head;
  return front_project(cq, d_qlat, n, d_qlat, w_up, w_qr, static_cast<int64_t>(dims->n_heads) * (w0 + dims->d_rope),
                       static_cast<int64_t>(dims->n_heads) * w0, part, rp, folded ? mla::kFrontQFolded : mla::kFrontQ,
                       st);
}

mla_status mla_q_project(const mla_dims* dims, const void* h, int64_t n, int32_t d_model, int32_t d_qlat,
                         const void* w_dq, const void* w_uq, const void* w_qr, const int32_t* q_pos, void* q_nope,
                         void* q_lat, void* workspace, size_t workspace_bytes, void* stream) {
  return q_project_impl(dims, h, n, d_model, d_qlat, w_dq, w_uq, w_qr, q_pos, q_nope, q_lat, workspace,
                        workspace_bytes, stream, false);
}

mla_status mla_q_project_folded(const mla_dims* dims, const void* h, int64_t n, int32_t d_model, int32_t d_qlat,
                                const void* w_dq, const void* w_fold, const void* w_qr, const int32_t* q_pos,
                                void* q_lat, void* workspace, size_t workspace_bytes, void* stream) {
  return q_project_impl(dims, h, n, d_model, d_qlat, w_dq, w_fold, w_qr, q_pos, nullptr, q_lat, workspace,
                        workspace_bytes, stream, true);
}

mla_status mla_fold_q_weights(const mla_dims* dims, int32_t d_qlat, const void* w_uq, const void* w_uk, void* w_fold,
                              void* stream) {
  g_err.clear();
  MLA_TRY(check_front(dims, 0, 32, d_qlat, true));
  if (w_uq == nullptr || w_uk == nullptr || w_fold == nullptr)
    return fail(MLA_ERR_INVALID_ARG, "w_uq, w_uk and w_fold must be non-NULL");
  mla::FoldParams p{static_cast<const mla::bf16_t*>(w_uq), static_cast<const mla::bf16_t*>(w_uk), static_cast<mla::bf16_t*>(w_fold),
                    dims->n_heads, dims->d_head, dims->d_latent, d_qlat};
  const hipError_t e = mla::launch_fold(p, as_stream(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "fold launch");
}

}  // extern "C"
