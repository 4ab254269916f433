// Host tier of the two-level cache: pinned host pools and the copy kernel that moves K/V
// rows between a device pool and a host pool ("SGLang: the tree, ...", ai.thesatyajit.com,
// "What the C++ tree is actually for": the tree keeps nodes on the GPU, on the CPU or both,
// and hands out copies to run as transactions).  The tree side lives in tree.cpp; this file
// owns the memory the copies touch.
//
// The copy is a gather/scatter over slot lists: every thread moves 16 bytes of one row of K
// and of V, reading or writing host memory over the bus directly (no staging buffer, no
// per-row memcpy), so a write-through or load back is one launch whatever the slot order.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <map>
#include <mutex>
#include <string>

#include "internal.h"

namespace {

// Rows src pool[src[r]] -> dst pool[dst[r]], K and V, 16 bytes per thread step.  Either pool
// pair may be pinned host memory.  A row whose slot lies outside its pool is skipped.
__global__ void copy_kv_kernel(uint4* __restrict__ dk, uint4* __restrict__ dv, const uint4* __restrict__ sk,
                               const uint4* __restrict__ sv, const int32_t* __restrict__ dst,
                               const int32_t* __restrict__ src, int64_t n, int row_chunks, int64_t dst_rows,
                               int64_t src_rows) {
  const int64_t total = n * row_chunks;
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < total; e += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = e / row_chunks, c = e % row_chunks;
    const int64_t d = dst[r], s = src[r];
    if (d < 0 || d >= dst_rows || s < 0 || s >= src_rows) continue;
    const int64_t from = s * row_chunks + c, to = d * row_chunks + c;
    const uint4 k = sk[from], v = sv[from];
    dk[to] = k;
    dv[to] = v;
  }
}

int grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  return int(std::min<int64_t>(std::max<int64_t>(g, 1), 65536));
}

int hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rs::fail(RS_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return RS_OK;
}

// Pinned host pools from rs_host_alloc: start -> bytes.  rs_copy_kv reads or writes host
// memory only inside these.
std::mutex g_host_mu;
std::map<uintptr_t, int64_t> g_host_pools;

// true if [p, p + bytes) lies inside one pinned pool of this library
bool in_host_pool(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  std::lock_guard<std::mutex> g(g_host_mu);
  auto it = g_host_pools.upper_bound(a);
  if (it == g_host_pools.begin()) return false;
  --it;
  return a >= it->first && a - it->first + uint64_t(bytes) <= uint64_t(it->second);
}

// a pool of `bytes` the copy kernel may touch: device memory, or inside a pinned host pool
int check_pool(const void* p, int64_t bytes, const char* name) {
  if (in_host_pool(p, bytes)) return RS_OK;
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    at.type = hipMemoryTypeUnregistered;
  }
  if (at.type != hipMemoryTypeDevice)
    return rs::fail(RS_E_INVAL, std::string("rs_copy_kv: ") + name +
                                    " is neither device memory nor inside a pool from rs_host_alloc");
  return RS_OK;
}
}  // namespace

extern "C" {

int rs_host_alloc(int64_t bytes, void** out) {
  if (bytes <= 0 || !out) return rs::fail(RS_E_INVAL, "rs_host_alloc: bad arguments");
  *out = nullptr;
  void* p = nullptr;
  if (hipHostMalloc(&p, size_t(bytes), hipHostMallocDefault) != hipSuccess || !p) {
    (void)hipGetLastError();
    return rs::fail(RS_E_NOSPACE, "rs_host_alloc: hipHostMalloc of " + std::to_string(bytes) + " bytes failed");
  }
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess || d != p) {
    (void)hipGetLastError();
    (void)hipHostFree(p);
    return rs::fail(RS_E_UNSUPPORTED, "rs_host_alloc: pinned memory is not mapped at its host address");
  }
  {
    std::lock_guard<std::mutex> g(g_host_mu);
    g_host_pools[reinterpret_cast<uintptr_t>(p)] = bytes;
  }
  *out = p;
  return RS_OK;
}

int rs_host_free(void* p) {
  if (!p) return RS_OK;
  {
    std::lock_guard<std::mutex> g(g_host_mu);
    auto it = g_host_pools.find(reinterpret_cast<uintptr_t>(p));
    if (it == g_host_pools.end()) return rs::fail(RS_E_INVAL, "rs_host_free: not a pool from rs_host_alloc");
    g_host_pools.erase(it);
  }
  return hipHostFree(p) == hipSuccess ? RS_OK : hip_check("rs_host_free");
}

int rs_copy_kv(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int32_t* dst_slots,
               const int32_t* src_slots, int64_t n, int64_t dst_rows, int64_t src_rows, int32_t Hkv, int32_t D,
               int32_t dtype, void* stream) {
  if (n < 0 || dst_rows < 0 || src_rows < 0 || Hkv <= 0 || D <= 0) return rs::fail(RS_E_INVAL, "rs_copy_kv: bad sizes");
  if (dtype != RS_DTYPE_F32 && dtype != RS_DTYPE_BF16) return rs::fail(RS_E_UNSUPPORTED, "rs_copy_kv: dtype");
  const int64_t row_bytes = int64_t(Hkv) * D * (dtype == RS_DTYPE_F32 ? 4 : 2);
  if (row_bytes % 16) return rs::fail(RS_E_UNSUPPORTED, "rs_copy_kv: a pool row must be a multiple of 16 bytes");
  if (n == 0) return RS_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !dst_slots || !src_slots)
    return rs::fail(RS_E_INVAL, "rs_copy_kv: null pointer");
  if ((reinterpret_cast<uintptr_t>(dst_k) | reinterpret_cast<uintptr_t>(dst_v) | reinterpret_cast<uintptr_t>(src_k) |
       reinterpret_cast<uintptr_t>(src_v)) & 15)
    return rs::fail(RS_E_INVAL, "rs_copy_kv: pools must be 16-byte aligned");
  // every pool must be memory the kernel can reach: device memory, or a pinned pool of this
  // library (other host memory would fault the kernel)
  int e;
  if ((e = check_pool(dst_k, dst_rows * row_bytes, "dst_k")) != RS_OK ||
      (e = check_pool(dst_v, dst_rows * row_bytes, "dst_v")) != RS_OK ||
      (e = check_pool(src_k, src_rows * row_bytes, "src_k")) != RS_OK ||
      (e = check_pool(src_v, src_rows * row_bytes, "src_v")) != RS_OK)
    return e;
  const int rc = int(row_bytes / 16);
  hipLaunchKernelGGL(copy_kv_kernel, dim3(grid_for(n * rc, 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(dst_k), static_cast<uint4*>(dst_v), static_cast<const uint4*>(src_k),
                     static_cast<const uint4*>(src_v), dst_slots, src_slots, n, rc, dst_rows, src_rows);
  return hip_check("rs_copy_kv");
}

}  // extern "C"
