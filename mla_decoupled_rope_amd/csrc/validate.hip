// Device-side check of the paging data a call is about to use, for the debug
// mode (MLA_DEBUG_VALIDATE=1).  The kernels themselves never fault on bad
// paging data -- they skip an out-of-range write and clamp an out-of-range
// read -- but the outputs are then unspecified.  This check runs first: one
// workgroup walks every (sequence, page) the call will read or write and every
// cache row it will write, and records the first entry out of range; the host
// reads the record back (synchronising the stream) and launches nothing else
// if it is bad.
#include <mutex>

#include "common.hpp"

namespace mla {

namespace {

constexpr int kCheckThreads = 1024;
constexpr int kMaxCheckDevices = 64;

// The record of the last check on this device: {kind, a, b, c, sum of the
// lengths, xor-hash of the lengths}.  Host code never passes the array's name
// to a kernel or a copy: its device address is looked up per device.
__device__ __align__(16) int32_t g_check[8];
void* g_check_ptr[kMaxCheckDevices];
std::once_flag g_check_once[kMaxCheckDevices];
hipError_t g_check_err[kMaxCheckDevices];

__global__ void __launch_bounds__(kCheckThreads) check_kernel(CheckParams p) {
  __shared__ int s_kind, s_a, s_b, s_c;
  __shared__ unsigned s_sum, s_hash;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_kind = 0;
    s_a = s_b = s_c = 0;
    s_sum = 0;
    s_hash = 0;
  }
  __syncthreads();
  auto report = [&](int kind, int a, int b, int c) {
    if (atomicCAS(&s_kind, 0, kind) == 0) {
      s_a = a;
      s_b = b;
      s_c = c;
    }
  };
  for (int b = tid; b < p.batch; b += kCheckThreads) {
    const int t = p.cu_q != nullptr ? p.q_start[b] + (p.cu_q[b + 1] - p.cu_q[b]) : p.seq_lens[b];
    atomicAdd(&s_sum, static_cast<unsigned>(t));
    atomicXor(&s_hash, (static_cast<unsigned>(t) * 2654435761u) ^ static_cast<unsigned>(b));
    if (t < 0 || static_cast<int64_t>(t) > static_cast<int64_t>(p.max_pages) * kPage) {
      report(kCheckLength, b, t, 0);
      continue;
    }
    const int pages = (t + kPage - 1) / kPage;
    const int32_t* row = p.block_table + static_cast<int64_t>(b) * p.max_pages;
    for (int pg = 0; pg < pages; ++pg) {
      const int id = row[pg];
      if (id < 0 || id >= p.num_pages) {
        report(kCheckPage, b, pg, id);
        break;
      }
    }
  }
  for (int64_t m = tid; m < p.n_kv; m += kCheckThreads) {
    const int b = p.kv_seq[m], pos = p.kv_pos[m];
    bool ok = b >= 0 && b < p.num_seqs && pos >= 0 && pos / kPage < p.max_pages;
    int id = -1;
    if (ok) {
      id = p.block_table[static_cast<int64_t>(b) * p.max_pages + pos / kPage];
      ok = id >= 0 && id < p.num_pages;
    }
    if (!ok) report(kCheckRow, static_cast<int>(m), b, pos);
  }
  __syncthreads();
  if (tid == 0) {
    g_check[0] = s_kind;
    g_check[1] = s_a;
    g_check[2] = s_b;
    g_check[3] = s_c;
    g_check[4] = static_cast<int32_t>(s_sum);
    g_check[5] = static_cast<int32_t>(s_hash);
  }
}

}  // namespace

hipError_t run_check(const CheckParams& p, int32_t* record, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxCheckDevices) return hipErrorInvalidDevice;
  std::call_once(g_check_once[dev], [dev] {
    void* ptr = nullptr;
    g_check_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_check));
    g_check_ptr[dev] = g_check_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_check_err[dev] != hipSuccess) return g_check_err[dev];
  hipLaunchKernelGGL(check_kernel, dim3(1), dim3(kCheckThreads), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(record, g_check_ptr[dev], 6 * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace mla
