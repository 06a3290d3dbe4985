// Producer: the rank-wide persistent grouped GEMM of the tile-signalling
// overlap paper (sec. 3.3.1). One launch covers every local expert through
// one tile worklist: tile t = (row band t / tiles_n, column tile t % tiles_n)
// with bands in the remote-first schedule order (sec. 3.2.2); workgroup i
// takes tiles i, i+g, i+2g, ... The expert of a band selects the weight
// pointer; no matrices are concatenated and nothing is relaunched per expert.
//
// gfx950 mapping: 256 threads = 4 waves in a 2x2 (or 1x4 / 2x2 for 64-row
// tiles) grid; v_mfma_f32_32x32x16_bf16 with fp32 accumulators; the k-loop
// stages 64-wide slices of A and B through two LDS buffers (register
// prefetch of the next slice while MFMAs run on the current one), with a
// 16-byte-chunk XOR swizzle so MFMA fragment reads are bank-conflict free.
//
// Epilogues:
//   EPI_PLAIN  C = A B^T (output projection y = h W2^T). With flags, after
//              the tile's stores every thread issues an agent-scope release
//              fence, the workgroup synchronises and one lane stores
//              flags[t] = epoch with release semantics (sec. 3.3.1:
//              store, fence, publish).
//   EPI_SILU   h = SiLU(x W1^T)                       (non-gated FFN)
//   EPI_GATED  h = SiLU(x W1^T) * (x W3^T); the B tile interleaves 32-row
//              blocks of W1 and W3 so each wave holds u and v of the same
//              h columns in registers.
#include "common.hpp"

namespace moe {

enum { EPI_PLAIN = 0, EPI_SILU = 1, EPI_GATED = 2 };

template <int BM, int BN>
struct Tile {
  static constexpr int BK = 64;
  static constexpr int WN = (BM >= 128) ? 2 : ((BN / 64) < 4 ? (BN / 64) : 4);
  static constexpr int WM = 4 / WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_LOADS = BM / 32, B_LOADS = BN / 32;   // 16-byte chunks per thread
  static constexpr int STAGE = (BM + BN) * BK;                 // bf16 elements per stage
  // at least 96 KiB so that one producer workgroup owns a CU
  static constexpr int LDS_ELEMS = (2 * STAGE > 49152) ? 2 * STAGE : 49152;
  static_assert(WM * WN == 4 && FM >= 1 && FN >= 1, "wave tiling");
};

struct GemmArgs {
  const uint16_t* A;           // [rows, K]
  const uint16_t* B0;          // [El, Nw, K]
  const uint16_t* B1;          // [El, Nw, K] (gated only)
  uint16_t* C;                 // [rows, Nout]
  const int32_t* meta;
  const int32_t* band_row0;
  const int32_t* band_expert;
  uint32_t* flags;             // output projection in overlap mode, else null
  uint32_t epoch;
  int K, Nw, Nout, tiles_n, bn_out;
};

// physical 16-byte chunk of logical chunk c in LDS row r
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ float silu_f32(float u) { return u / (1.0f + __expf(-u)); }

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm(const GemmArgs a) {
  using C = Tile<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int n_tiles = a.meta[META_NBANDS] * a.tiles_n;
  const int K = a.K;
  const int nk = K / C::BK;
  const int cc = tid & 7;    // logical 16-byte chunk this thread loads
  const int rr = tid >> 3;   // first row this thread loads (rows rr + 32 i)

  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int band = tile / a.tiles_n;
    const int tn = tile - band * a.tiles_n;
    const int row0 = a.band_row0[band];
    const int e = a.band_expert[band];
    const uint16_t* asrc = a.A + (size_t)(row0 + rr) * K + cc * 8;
    const uint16_t* bsrc[C::B_LOADS];
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
      int wrow;
      const uint16_t* base;
      if constexpr (EPI == EPI_GATED) {
        base = ((i & 1) ? a.B1 : a.B0) + (size_t)e * a.Nw * K;
        wrow = tn * (BN / 2) + (i >> 1) * 32 + rr;
      } else {
        base = a.B0 + (size_t)e * a.Nw * K;
        wrow = tn * BN + i * 32 + rr;
      }
      bsrc[i] = base + (size_t)wrow * K + cc * 8;
    }

    u32x4 ra[C::A_LOADS], rb[C::B_LOADS];
    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    auto gload = [&](int kt) {
      const size_t ko = (size_t)kt * C::BK;
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i)
        ra[i] = *reinterpret_cast<const u32x4*>(asrc + (size_t)i * 32 * K + ko);
#pragma unroll
      for (int i = 0; i < C::B_LOADS; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bsrc[i] + ko);
    };
    auto sstore = [&](int buf) {
      uint16_t* As = lds + buf * C::STAGE;
      uint16_t* Bs = As + BM * C::BK;
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i) {
        const int r = rr + 32 * i;
        *reinterpret_cast<u32x4*>(As + r * C::BK + swz(r, cc) * 8) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < C::B_LOADS; ++i) {
        const int r = rr + 32 * i;
        *reinterpret_cast<u32x4*>(Bs + r * C::BK + swz(r, cc) * 8) = rb[i];
      }
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      const uint16_t* As = lds + cur * C::STAGE;
      const uint16_t* Bs = As + BM * C::BK;
#pragma unroll
      for (int kk = 0; kk < C::BK / 16; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
        bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          const int r = wm * C::WTM + i * 32 + (lane & 31);
          af[i] = *reinterpret_cast<const bf16x8*>(As + r * C::BK + swz(r, ch) * 8);
        }
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int r = wn * C::WTN + j * 32 + (lane & 31);
          bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + r * C::BK + swz(r, ch) * 8);
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) sstore(cur ^ 1);
      __syncthreads();
    }

    // epilogue: 32x32 accumulator layout: lane l holds column l%32, rows
    // 8*(q/4) + 4*(l/32) + q%4 for q = 0..15
    const int ncol = lane & 31;
    const int mrow = (lane >> 5) * 4;
    if constexpr (EPI == EPI_GATED) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int p = 0; p < C::FN / 2; ++p) {
          const int col = tn * (BN / 2) + wn * (C::WTN / 2) + p * 32 + ncol;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int m = wm * C::WTM + i * 32 + (q >> 2) * 8 + mrow + (q & 3);
            const float u = acc[i][2 * p][q], v = acc[i][2 * p + 1][q];
            a.C[(size_t)(row0 + m) * a.Nout + col] = f32_to_bf16_rne(silu_f32(u) * v);
          }
        }
    } else {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int col = tn * BN + wn * C::WTN + j * 32 + ncol;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int m = wm * C::WTM + i * 32 + (q >> 2) * 8 + mrow + (q & 3);
            float v = acc[i][j][q];
            if constexpr (EPI == EPI_SILU) v = silu_f32(v);
            a.C[(size_t)(row0 + m) * a.Nout + col] = f32_to_bf16_rne(v);
          }
        }
      if (a.flags != nullptr) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0)
          __hip_atomic_store(a.flags + tile, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <int BM, int BN, int EPI>
static hipError_t launch_t(const GemmArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((k_gemm<BM, BN, EPI>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int EPI>
static hipError_t dispatch(const GemmArgs& a, int bm, int bn, int grid, hipStream_t st) {
  if (bm == 256 && bn == 256) return launch_t<256, 256, EPI>(a, grid, st);
  if (bm == 256 && bn == 128) return launch_t<256, 128, EPI>(a, grid, st);
  if (bm == 128 && bn == 256) return launch_t<128, 256, EPI>(a, grid, st);
  if (bm == 128 && bn == 128) return launch_t<128, 128, EPI>(a, grid, st);
  if (bm == 64 && bn == 256) return launch_t<64, 256, EPI>(a, grid, st);
  if (bm == 64 && bn == 128) return launch_t<64, 128, EPI>(a, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm1(const Geometry& g, const uint16_t* x_perm, const uint16_t* w1,
                        const uint16_t* w3, uint16_t* h, const moe_plan_t& p, int grid,
                        hipStream_t st) {
  GemmArgs a{};
  a.A = x_perm;
  a.B0 = w1;
  a.B1 = w3;
  a.C = h;
  a.meta = p.meta;
  a.band_row0 = p.band_row0;
  a.band_expert = p.band_expert;
  a.flags = nullptr;
  a.epoch = 0;
  a.K = g.H;
  a.Nw = g.F;
  a.Nout = g.F;
  a.tiles_n = g.tiles1;
  a.bn_out = g.bn1_out;
  return g.gated ? dispatch<EPI_GATED>(a, g.tb_m, g.bn1, grid, st)
                 : dispatch<EPI_SILU>(a, g.tb_m, g.bn1, grid, st);
}

hipError_t launch_gemm2(const Geometry& g, const uint16_t* h, const uint16_t* w2, uint16_t* y,
                        const moe_plan_t& p, uint32_t* flags, uint32_t epoch, int grid,
                        hipStream_t st) {
  GemmArgs a{};
  a.A = h;
  a.B0 = w2;
  a.B1 = nullptr;
  a.C = y;
  a.meta = p.meta;
  a.band_row0 = p.band_row0;
  a.band_expert = p.band_expert;
  a.flags = flags;
  a.epoch = epoch;
  a.K = g.F;
  a.Nw = g.H;
  a.Nout = g.H;
  a.tiles_n = g.tiles2;
  a.bn_out = g.bn2;
  return dispatch<EPI_PLAIN>(a, g.tb_m, g.bn2, grid, st);
}

}  // namespace moe
