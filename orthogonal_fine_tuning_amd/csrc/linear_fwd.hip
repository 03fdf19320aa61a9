// Forward of the dense OFT linear layer: y = rot_R(x . dequant(W0)^T).
//
// Orbit pages: the base weight stays at deployment precision (chooseai.io
// release news, "Technical principles") and fused projections get one
// independent rotation per sub-projection, applied by custom split-projection
// kernels ("Five design features of the adapter-first architecture").
//
// One launch with the rotation epilogue: gemm_nt_dma_kernel (gemm_nt_dma.h)
// for bf16 activations, gemm_nt_kernel (gemm_nt.h) for fp32 ones (converted
// to bf16 on the way into LDS), gemm_nt_skinny_kernel (gemm_skinny.h) for
// decode batches of at most 64 tokens.  A 32-channel accumulator group is
// exactly one b = 32 block (or two b = 16 blocks), and blocks never straddle
// projection segments, so every segment gets its own rotation with no extra
// pass over HBM.
#include "gemm_nt.h"
#include "gemm_nt_dma.h"
#include "gemm_nt_hl.h"
#include "gemm_skinny.h"
#include "oft_launch.h"
#include "oft_prof.h"

namespace oft {
namespace {

constexpr int FWD_BM = 256;
constexpr int FWD_NBUF = 1;

// EPI: EPI_ROT (the adapted layer) or EPI_BASE (the frozen base alone)
template <bool XF32, int WF, int B, int EPI = EPI_ROT>
hipError_t launch_fwd_t(const DenseArgs& a, const void* x, const uint8_t* wc, const void* ws,
                        const uint16_t* Rops, void* y, hipStream_t st) {
  constexpr bool FP8 = WF == WF_FP8;
  if constexpr (!XF32) {
    if (a.M <= 64) {  // few tokens: weight stream through the deep copy ring
      NtArgs p{};
      p.a = x;
      p.lda = a.K;
      p.wc = wc;
      p.ws = ws;
      p.rops = Rops;
    p.rops_alt = a.rops_alt;
    p.rops_sel = a.rops_sel;
      p.out = y;
      p.ldo = a.N;
      p.M = a.M;
      p.K = a.K;
      p.N = a.N;
      p.g = a.g;
      const dim3 grid((a.N + ntd::DEC_BN - 1) / ntd::DEC_BN, 1);
      if (!FP8 && a.K % 256 == 0)  // 4-bit: whole-line weight copies on 256-wide steps, 16 waves
        hipLaunchKernelGGL((gemm_nt_dec16_kernel<B, EPI, FP8 ? WF_INT4 : WF>), grid, dim3(1024), 0, st, p);
      else
        hipLaunchKernelGGL((gemm_nt_dec_kernel<WF, B, EPI>), grid, dim3(ntd::DEC_NTHR), 0, st, p);
      return hipGetLastError();
    }
  }
  if (a.M <= 64 && a.K % 256 == 0) {  // few tokens, fp32 activations: weight-streaming kernel
    NtArgs p{};
    p.a = x;
    p.lda = a.K;
    p.wc = wc;
    p.ws = ws;
    p.rops = Rops;
    p.rops_alt = a.rops_alt;
    p.rops_sel = a.rops_sel;
    p.out = y;
    p.ldo = a.N;
    p.M = a.M;
    p.K = a.K;
    p.N = a.N;
    p.g = a.g;
    constexpr int TN = 2;
    if (a.N % (32 * TN) == 0) {
      hipLaunchKernelGGL((gemm_nt_skinny_kernel<XF32, WF, B, XF32, TN, EPI>), dim3(a.N / (32 * TN), 1), dim3(256),
                         0, st, p);
    } else {
      hipLaunchKernelGGL((gemm_nt_skinny_kernel<XF32, WF, B, XF32, 1, EPI>), dim3(a.N / 32, 1), dim3(256), 0, st,
                         p);
    }
    return hipGetLastError();
  }
  NtArgs p{};
  p.a = x;
  p.lda = a.K;
  p.wc = wc;
  p.ws = ws;
  p.rops = Rops;
  p.rops_alt = a.rops_alt;
  p.rops_sel = a.rops_sel;
  p.out = y;
  p.ldo = a.N;
  p.M = a.M;
  p.K = a.K;
  p.N = a.N;
  p.g = a.g;
  if constexpr (!XF32) {
    if (a.K % ntd::BK == 0) {
      const int nt = (a.N + ntd::BN - 1) / ntd::BN;
      const int bm = pick_token_tile(nt, a.M, num_cus(), 192);
      if (bm == 192 && FP8 && a.K % 128 == 0)  // FP8: 128-wide K steps
        hipLaunchKernelGGL((gemm_nt_dma_kernel<WF_FP8, B, 192, EPI, false, false, 128>),
                           dim3(nt, (a.M + 191) / 192), dim3(ntd::NTHR), 0, st, p);
      else if (bm == 192)
        hipLaunchKernelGGL((gemm_nt_dma_kernel<WF, B, 192, EPI, false>), dim3(nt, (a.M + 191) / 192),
                           dim3(ntd::NTHR), 0, st, p);
      else {
        bool hl = false;
        if constexpr (wf_4bit(WF)) {
          if (a.K % 128 == 0) {  // weight stages of two K steps (half-line copies)
            hipLaunchKernelGGL((gemm_nt_hl_kernel<WF, B, EPI, false>), dim3(nt, (a.M + 127) / 128),
                               dim3(nth::NTHR), 0, st, p);
            hl = true;
          }
        }
        if (!hl)
          hipLaunchKernelGGL((gemm_nt_dma_kernel<WF, B, 128, EPI, false>), dim3(nt, (a.M + 127) / 128),
                             dim3(ntd::NTHR), 0, st, p);
      }
      return hipGetLastError();
    }
  }
  dim3 grid((a.N + nt::BN - 1) / nt::BN, (a.M + FWD_BM - 1) / FWD_BM);
  hipLaunchKernelGGL((gemm_nt_kernel<FWD_BM, XF32, WF, B, EPI, false, XF32, FWD_NBUF>), grid, dim3(256), 0,
                     st, p);
  return hipGetLastError();
}

}  // namespace

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

hipError_t launch_linear_fwd(const DenseArgs& a, const void* x, const uint8_t* wc, const void* ws,
                             const uint16_t* Rops, void* y, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  ProfScope prof(st, "dense.fwd");
#define OFT_FWD_CASE(XF, WFV, BB) \
  if (a.xf32 == XF && a.wf == WFV && a.b == BB) return launch_fwd_t<XF, WFV, BB>(a, x, wc, ws, Rops, y, st);
#define OFT_FWD_B(XF, WFV) OFT_FWD_CASE(XF, WFV, 32) OFT_FWD_CASE(XF, WFV, 16)
  OFT_FWD_B(false, WF_INT4)
  OFT_FWD_B(false, WF_FP8)
  OFT_FWD_B(false, WF_FP4)
  OFT_FWD_B(true, WF_INT4)
  OFT_FWD_B(true, WF_FP8)
  OFT_FWD_B(true, WF_FP4)
#undef OFT_FWD_B
#undef OFT_FWD_CASE
  return hipErrorInvalidValue;
}

// ---- double-buffered adapter slots ----------------------------------------
// One thread each.  The state {active slot, its version} is one 64-bit word:
// the switch stores it and the latch loads it with single device-scope
// atomics, so a latch sees either the old pair or the new one, never a mix.
// The rotation pack needs no fence of its own here: the Cayley build before
// the switch has completed (and released its writes at its kernel boundary)
// before the switch can store, and the forward kernels start after the
// latch, with the acquire at their own kernel boundary.
__global__ __launch_bounds__(64) void slots_switch_kernel(int* state, int slot, int version) {
  if (threadIdx.x != 0) return;
  const unsigned long long w = (unsigned long long)(unsigned)slot | ((unsigned long long)(unsigned)version << 32);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(state), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(64) void slots_latch_kernel(const int* state, int* latch) {
  if (threadIdx.x != 0) return;
  const unsigned long long w =
      __hip_atomic_load(reinterpret_cast<const unsigned long long*>(state), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  latch[0] = (unsigned)w == 1u ? 1 : 0;
  latch[1] = (int)(unsigned)(w >> 32);
}

hipError_t launch_slots_switch(int* state, int slot, int version, hipStream_t st) {
  hipLaunchKernelGGL(slots_switch_kernel, dim3(1), dim3(64), 0, st, state, slot, version);
  return hipGetLastError();
}

hipError_t launch_linear_fwd_slots(const DenseArgs& a, const void* x, const uint8_t* wc, const void* ws,
                                   const uint16_t* R0, const uint16_t* R1, const int* state, int* latch, void* y,
                                   hipStream_t st) {
  {
    ProfScope prof(st, "dense.slots_latch");
    hipLaunchKernelGGL(slots_latch_kernel, dim3(1), dim3(64), 0, st, state, latch);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.M == 0) return err;
  DenseArgs s = a;
  // the second pack as an element offset from the first, taken on the
  // integer addresses (both packs live in the one flat device address space
  // and are 16-byte aligned)
  s.rops_alt = (long)((intptr_t)R1 - (intptr_t)R0) / (long)sizeof(uint16_t);
  s.rops_sel = latch;
  return launch_linear_fwd(s, x, wc, ws, R0, y, st);
}

// The frozen base alone (R = I): y = x . dequant(W0)^T, the same kernels with
// the rotation epilogue left out (the block size plays no part)
hipError_t launch_linear_fwd_base(const DenseArgs& a, const void* x, const uint8_t* wc, const void* ws, void* y,
                                  hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  ProfScope prof(st, "dense.fwd_base");
#define OFT_BASE_CASE(XF, WFV) \
  if (a.xf32 == XF && a.wf == WFV) return launch_fwd_t<XF, WFV, 32, EPI_BASE>(a, x, wc, ws, nullptr, y, st);
  OFT_BASE_CASE(false, WF_INT4)
  OFT_BASE_CASE(false, WF_FP8)
  OFT_BASE_CASE(false, WF_FP4)
  OFT_BASE_CASE(true, WF_INT4)
  OFT_BASE_CASE(true, WF_FP8)
  OFT_BASE_CASE(true, WF_FP4)
#undef OFT_BASE_CASE
  return hipErrorInvalidValue;
}

}  // namespace oft
