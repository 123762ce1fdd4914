// Streaming-read reference for the decode measurements: how fast this GPU
// reads pages of a pool, with nothing computed.  It is not part of the
// decode path; the benchmark reports its rate beside the decode kernels'.
//
// A workgroup of 8 waves reads `pages_per_wg` pages of `page_bytes` bytes
// (a multiple of 1024), taken in the order a shuffled page table lists them,
// the whole page at a time: wave w loads 16 bytes per lane at byte
// 1024 i + 16 lane of the page for i = w, w + 8, ...  The loads of a page
// are all issued before any is used, and the workgroup keeps one page ahead.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWaves = 8;
constexpr int kMaxInst = 8;   // 1 KB loads per wave per page: pages of up to 64 KB

__global__ __launch_bounds__(kWaves * 64) void page_read_kernel(const uint8_t* __restrict__ pool,
                                                                const int32_t* __restrict__ pages, uint32_t npages,
                                                                uint32_t pages_per_wg, uint32_t page_bytes,
                                                                uint32_t* __restrict__ sink) {
  __shared__ int32_t pid[256];
  const uint32_t first = blockIdx.x * pages_per_wg;
  if (first >= npages) return;
  const uint32_t cnt = min(pages_per_wg, npages - first);
  for (uint32_t i = threadIdx.x; i < cnt; i += blockDim.x) pid[i] = pages[first + i];
  __syncthreads();
  const uint32_t w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t ninst = page_bytes / 1024;
  uint4 acc = {0u, 0u, 0u, 0u};
  uint4 buf[2][kMaxInst];
  auto load = [&](uint32_t i, uint4(&b)[kMaxInst]) {
    const uint8_t* base = pool + uint64_t(uint32_t(pid[min(i, cnt - 1)])) * page_bytes + lane * 16;
#pragma unroll
    for (int k = 0; k < kMaxInst; ++k) {
      const uint32_t ins = w + k * kWaves;
      if (ins < ninst) b[k] = *reinterpret_cast<const uint4*>(base + ins * 1024);
    }
  };
  load(0, buf[0]);
  for (uint32_t i = 0; i < cnt; i += 2) {
    load(i + 1, buf[1]);
#pragma unroll
    for (int k = 0; k < kMaxInst; ++k)
      if (w + k * kWaves < ninst) { acc.x ^= buf[0][k].x; acc.y ^= buf[0][k].y; acc.z ^= buf[0][k].z; acc.w ^= buf[0][k].w; }
    load(i + 2, buf[0]);
#pragma unroll
    for (int k = 0; k < kMaxInst; ++k)
      if (w + k * kWaves < ninst && i + 1 < cnt) {
        acc.x ^= buf[1][k].x; acc.y ^= buf[1][k].y; acc.z ^= buf[1][k].z; acc.w ^= buf[1][k].w;
      }
  }
  // the xor of everything read, so that no load can be dropped
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == 0x9E3779B9u) sink[blockIdx.x] = v;
}

// The same pages read straight into LDS (global_load_lds_dwordx4: 16 bytes
// per lane, M0 the LDS address of the instruction's 1 KB block) through a
// ring of three page stages: a workgroup keeps two pages in flight, and no
// VGPR holds a load.  Each wave issues its share of a page's 1 KB blocks;
// before using stage i a wave waits until only its loads of the later
// stage remain in flight, then the workgroup meets.
__device__ __forceinline__ void lds_load16(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_loads() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

constexpr int kStages = 3;

__global__ __launch_bounds__(kWaves * 64) void page_read_lds_kernel(const uint8_t* __restrict__ pool,
                                                                    const int32_t* __restrict__ pages,
                                                                    uint32_t npages, uint32_t pages_per_wg,
                                                                    uint32_t page_bytes, uint32_t* __restrict__ sink) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  __shared__ int32_t pid[256];
  const uint32_t first = blockIdx.x * pages_per_wg;
  if (first >= npages) return;
  const uint32_t cnt = min(pages_per_wg, npages - first);
  for (uint32_t i = threadIdx.x; i < cnt; i += blockDim.x) pid[i] = pages[first + i];
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ninst = page_bytes / 1024;
  const uint32_t mine = (ninst + kWaves - 1 - w) / kWaves;  // this wave's blocks of a page (<= kMaxInst)
  // the ring's LDS byte address (an LDS-space pointer's value)
  const uint32_t ring_base =
      uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)ring));
  auto issue = [&](uint32_t i) {  // page i of the run -> stage i % kStages (past the end: the last page again)
    const uint32_t pg = uint32_t(__builtin_amdgcn_readfirstlane(pid[min(i, cnt - 1)]));
    const uint8_t* base = pool + uint64_t(pg) * page_bytes;
    const uint32_t st = ring_base + (i % kStages) * page_bytes;
    for (uint32_t ins = w; ins < ninst; ins += kWaves) lds_load16(base, ins * 1024 + lane * 16, st + ins * 1024);
  };
  for (uint32_t i = 0; i + 1 < kStages; ++i) issue(i);
  uint32_t acc = 0;
  for (uint32_t i = 0; i < cnt; ++i) {
    switch (mine) {  // stage i done: this wave's loads of the one later stage may stay in flight
      case 0: break;
      case 1: wait_loads<1>(); break;
      case 2: wait_loads<2>(); break;
      case 3: wait_loads<3>(); break;
      case 4: wait_loads<4>(); break;
      case 5: wait_loads<5>(); break;
      case 6: wait_loads<6>(); break;
      case 7: wait_loads<7>(); break;
      default: wait_loads<8>(); break;
    }
    __syncthreads();  // every wave's blocks of stage i are in LDS; stage i - 1 is free
    issue(i + kStages - 1);
    const uint32_t* stg = reinterpret_cast<const uint32_t*>(ring + (i % kStages) * page_bytes);
    acc ^= stg[threadIdx.x % (page_bytes / 4)];
  }
  wait_loads<0>();
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads npages pages of page_bytes bytes (pages[i] < pool pages; 16-byte
// aligned pool) `reps` times on `stream` and returns the elapsed seconds of
// the timed repetitions (one untimed repetition first), or a negative value on
// an invalid argument or a HIP error.  Synchronizes the host.
double kvq_probe_page_read(const void* pool, const int32_t* pages, uint32_t npages, uint32_t page_bytes,
                           uint32_t pages_per_wg, uint32_t reps, uint32_t* sink, void* stream) {
  if (!pool || !pages || !sink || npages == 0 || reps == 0 || page_bytes == 0 || page_bytes % 1024 ||
      page_bytes > 1024u * kWaves * kMaxInst || pages_per_wg == 0 || pages_per_wg > 256)
    return -1.0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint32_t grid = (npages + pages_per_wg - 1) / pages_per_wg;
  auto launch = [&] {
    hipLaunchKernelGGL(page_read_kernel, dim3(grid), dim3(kWaves * 64), 0, st, static_cast<const uint8_t*>(pool),
                       pages, npages, pages_per_wg, page_bytes, sink);
  };
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -2.0;
  launch();
  hipEventRecord(a, st);
  for (uint32_t r = 0; r < reps; ++r) launch();
  hipEventRecord(b, st);
  const hipError_t e = hipEventSynchronize(b);
  float ms = 0.0f;
  hipEventElapsedTime(&ms, a, b);
  hipEventDestroy(a);
  hipEventDestroy(b);
  if (e != hipSuccess || hipGetLastError() != hipSuccess) return -3.0;
  return double(ms) * 1e-3;
}

// As kvq_probe_page_read, with the pages read straight into LDS (page_bytes
// at most 53248: three stages fit in a CU's LDS).
double kvq_probe_page_read_lds(const void* pool, const int32_t* pages, uint32_t npages, uint32_t page_bytes,
                               uint32_t pages_per_wg, uint32_t reps, uint32_t* sink, void* stream) {
  if (!pool || !pages || !sink || npages == 0 || reps == 0 || page_bytes == 0 || page_bytes % 1024 ||
      page_bytes * kStages > 160u * 1024u || page_bytes > 1024u * kWaves * kMaxInst || pages_per_wg == 0 ||
      pages_per_wg > 256)
    return -1.0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint32_t grid = (npages + pages_per_wg - 1) / pages_per_wg;
  const size_t lds = size_t(page_bytes) * kStages;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(page_read_lds_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
    return -2.0;
  auto launch = [&] {
    hipLaunchKernelGGL(page_read_lds_kernel, dim3(grid), dim3(kWaves * 64), lds, st,
                       static_cast<const uint8_t*>(pool), pages, npages, pages_per_wg, page_bytes, sink);
  };
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -2.0;
  launch();
  hipEventRecord(a, st);
  for (uint32_t r = 0; r < reps; ++r) launch();
  hipEventRecord(b, st);
  const hipError_t e = hipEventSynchronize(b);
  float ms = 0.0f;
  hipEventElapsedTime(&ms, a, b);
  hipEventDestroy(a);
  hipEventDestroy(b);
  if (e != hipSuccess || hipGetLastError() != hipSuccess) return -3.0;
  return double(ms) * 1e-3;
}

}  // extern "C"
