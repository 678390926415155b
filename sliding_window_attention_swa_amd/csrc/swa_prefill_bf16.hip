// Banded sliding-window attention prefill for bfloat16 on gfx950 matrix cores.
//
// What is computed (robocikowo glossary "Sliding Window Attention", opening
// definition; Ultralytics glossary, section "Come cresce la finestra con la
// profondita"): out_i = softmax over the keys j of i's window of
// scale * q_i . k_j, applied to the v_j.  Causal window 0 <= i-j <= W-1,
// symmetric window |i-j| <= floor(W/2), both clipped to [0, T).
//
// Structure (one workgroup = 128 query rows of one query head, 4 waves of 32
// rows each; key tiles of 64 rows):
//   * only the key tiles that intersect the union of the block's windows are
//     visited, so the work is O(T * W * d) and no [T, T] matrix exists;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K tile from LDS as the A
//     operand, the wave's Q rows held in registers as the B operand), so each
//     lane owns one query row of the score tile and the row statistics need
//     only one cross-lane exchange (lane l with lane l^32);
//   * the out-of-window mask is applied only on tiles that cross a window
//     edge or the end of the sequence;
//   * online softmax in fp32 with a lazily updated reference maximum: the
//     accumulators are rescaled only when a row's maximum grows by more than
//     2^8, which keeps every exponent <= 2^8 and changes only rounding;
//   * P is rounded to bf16 and used straight from the score registers as the
//     B operand of O^T += V^T P^T; V^T comes from the natural [key][dim] LDS
//     tile through the gfx950 transposing LDS read (ds_read_b64_tr_b16);
//   * K/V tiles are double-buffered: the next tile's global loads are in
//     flight while the current one is consumed, one barrier per tile;
//   * grouped-query heads: query head h reads KV head h / (Hq / Hkv); the
//     workgroup order keeps the heads of one group and neighbouring query
//     blocks on the same XCD so their K/V tiles are shared through its L2.

#include "swa_device.h"
#include "swa_launch.h"

namespace swa {
namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // key rows per tile
constexpr int kThreads = 256;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kNegBig = -1.0e30f;        // finite "no maximum yet"

template <int D>
struct Geo {
  static constexpr int PITCH = D + 8;           // LDS row pitch (elements): 16 B pad
  static constexpr int TILE = kBN * PITCH;      // elements in one K or V tile
  static constexpr int KS = D / 16;             // k-steps of the QK^T contraction
  static constexpr int MD = D / 32;             // 32-dim blocks of the output
  static constexpr int TPR = D / 8;             // copy threads per row (16 B each)
  static constexpr int RPI = kThreads / TPR;    // rows per copy instruction
  static constexpr int NLD = kBN / RPI;         // copy instructions per tile
  static constexpr int LDS_BYTES = 2 * 2 * TILE * 2;
};

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ out, int T, int W, int Hq, int Hkv, float scale_log2, int n_qtiles) {
  using Gm = Geo<D>;
  constexpr int PITCH = Gm::PITCH, TILE = Gm::TILE, KS = Gm::KS, MD = Gm::MD;
  constexpr int TPR = Gm::TPR, RPI = Gm::RPI, NLD = Gm::NLD;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * 2 * TILE];  // [stage][K|V][kBN][PITCH]

  // ---- which (query head, query block) this workgroup owns
  const int G = Hq / Hkv;
  int id = blockIdx.x;
  const int nwg = gridDim.x;
  // Consecutive workgroup ids are dealt round-robin to the 8 XCDs; regroup
  // them so that each XCD receives a contiguous range of logical ids.
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int hg = id % G;
  const int rest = id / G;
  const int qt = rest % n_qtiles;
  const int kvh = rest / n_qtiles;
  const int h = kvh * G + hg;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;  // which 8 of the 16 contraction elements this lane holds
  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + (lane & 31);  // the query row this lane owns

  const __bf16* qh = q + (size_t)h * T * D;
  const __bf16* kh = k + (size_t)kvh * T * D;
  const __bf16* vh = v + (size_t)kvh * T * D;

  const int hw = W >> 1;
  int lo, hi;
  if (MODE == 0) {
    lo = max(0, q0 - W + 1);
    hi = min(T - 1, q0 + kBM - 1);
  } else {
    lo = max(0, q0 - hw);
    hi = min(T - 1, q0 + kBM - 1 + hw);
  }
  const int kt0 = lo / kBN, kt1 = hi / kBN;

  // this wave's rows and key range
  const bool wave_active = qw0 < T;
  const int qlast = min(qw0 + 31, T - 1);
  const int wlo = (MODE == 0) ? max(0, qw0 - W + 1) : max(0, qw0 - hw);
  const int whi = (MODE == 0) ? qlast : min(T - 1, qlast + hw);

  // ---- Q rows as B operands (one per k-step), zero beyond the sequence
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (qi < T) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qh + (size_t)qi * D + ks * 16 + half * 8);
    } else {
      qf[ks] = bf16x8{};
    }
  }

  // ---- global -> register -> LDS tile copy
  uint4 kreg[NLD], vreg[NLD];
  const int crow = tid / TPR;
  const int ccol = (tid % TPR) * 8;
  auto load_tile = [&](int kt) {
    const int kbase = kt * kBN;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int key = kbase + i * RPI + crow;
      if (key < T) {
        kreg[i] = *reinterpret_cast<const uint4*>(kh + (size_t)key * D + ccol);
        vreg[i] = *reinterpret_cast<const uint4*>(vh + (size_t)key * D + ccol);
      } else {
        kreg[i] = make_uint4(0, 0, 0, 0);
        vreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int stage) {
    __bf16* Ks = smem + stage * 2 * TILE;
    __bf16* Vs = Ks + TILE;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = i * RPI + crow;
      *reinterpret_cast<uint4*>(Ks + r * PITCH + ccol) = kreg[i];
      *reinterpret_cast<uint4*>(Vs + r * PITCH + ccol) = vreg[i];
    }
  };

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = f32x16{};
  float m_ref = kNegBig;  // reference maximum (log2 domain) of this lane's row
  float l_part = 0.f;     // this lane's share of the row's exponential sum

  // source-lane addressing of the transposing V read (see the PV step)
  const int tr_s = lane & 15;
  const int tr_g = lane >> 4;
  const int tr_row = 4 * (tr_g >> 1) + (tr_s >> 2);
  const int tr_col = 16 * (tr_g & 1) + 4 * (tr_s & 3);

  load_tile(kt0);
  store_tile(0);
  __syncthreads();

  for (int kt = kt0; kt <= kt1; ++kt) {
    const int stage = (kt - kt0) & 1;
    if (kt < kt1) load_tile(kt + 1);
    const int k0 = kt * kBN;
    const bool relevant = wave_active && k0 <= whi && k0 + kBN - 1 >= wlo;
    if (relevant) {
      const __bf16* Ks = smem + stage * 2 * TILE;
      const __bf16* Vs = Ks + TILE;

      // ---- S^T tile: 64 keys x 32 queries, two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
        const __bf16* krow = Ks + (mb * 32 + (lane & 31)) * PITCH + half * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + ks * 16);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mb], 0, 0, 0);
        }
      }

      // ---- scale into the log2 domain; mask tiles that cross an edge
      bool full;
      if (MODE == 0) {
        full = (k0 + kBN - 1 <= qw0) && (k0 >= qlast - W + 1) && (k0 + kBN <= T);
      } else {
        full = (k0 >= qlast - hw) && (k0 + kBN - 1 <= qw0 + hw) && (k0 + kBN <= T);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][r] *= scale_log2;
      }
      if (!full) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const int diff = qi - key;
            bool ok = key < T;
            if (MODE == 0) {
              ok = ok && diff >= 0 && diff < W;
            } else {
              ok = ok && diff >= -hw && diff <= hw;
            }
            if (!ok) s[mb][r] = -INFINITY;
          }
        }
      }

      // ---- row maximum (this lane's 32 scores, then the partner lane's)
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      mx = wave_max_xor32(mx);

      const bool grow = mx > m_ref + kRescaleThreshold;
      if (__ballot(grow)) {
        const float m_new = grow ? mx : m_ref;
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        l_part *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md) {
#pragma unroll
          for (int r = 0; r < 16; ++r) o[md][r] *= alpha;
        }
      }

      // ---- probabilities, row sum, bf16 B operands of the PV product
      bf16x8 pb[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[mb][r] - m_ref);
          s[mb][r] = p;
          l_part += p;
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(s[mb][8 * k2 + 2 * e], s[mb][8 * k2 + 2 * e + 1]);
          pb[mb][k2] = __builtin_bit_cast(bf16x8, w);
        }
      }

      // ---- O^T += V^T P^T.  Element j of pb[mb][k2] in lane l holds key
      // mb*32 + 16*k2 + 8*(j/4) + 4*(l/32) + j%4.  The A operand must hold
      // V at those keys for dim 32*md + l%32; two transposing reads give
      // exactly that: within each 16-lane group, lane i receives component
      // i%4 of the 8 bytes addressed by lane 4*j + i/4, and each source lane
      // addresses 4 consecutive dims of one key row.
#pragma unroll
      for (int md = 0; md < MD; ++md) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const __bf16* src = Vs + (mb * 32 + 16 * k2 + tr_row) * PITCH + 32 * md + tr_col;
            const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src));
            const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + 8 * PITCH));
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            const i16x8 a16 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            const bf16x8 a = __builtin_bit_cast(bf16x8, a16);
            o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[mb][k2], o[md], 0, 0, 0);
          }
        }
      }
    }
    if (kt < kt1) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: divide by the row sum, round to bf16, store
  if (qi < T) {
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    const float inv = 1.0f / l_tot;
    __bf16* orow = out + ((size_t)h * T + qi) * D;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int dim = 32 * md + 8 * rq + 4 * half;
        uint2 w;
        w.x = pack_bf16x2(o[md][4 * rq + 0] * inv, o[md][4 * rq + 1] * inv);
        w.y = pack_bf16x2(o[md][4 * rq + 2] * inv, o[md][4 * rq + 3] * inv);
        *reinterpret_cast<uint2*>(orow + dim) = w;
      }
    }
  }
}

template <int D, int MODE>
hipError_t launch(const void* q, const void* k, const void* v, void* out, int T, int W, int Hq,
                  int Hkv, float scale, hipStream_t stream) {
  const int n_qtiles = (T + kBM - 1) / kBM;
  const long long nwg = (long long)n_qtiles * Hq;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, MODE>), dim3((unsigned)nwg), dim3(kThreads), 0,
                     stream, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), static_cast<__bf16*>(out), T, W, Hq, Hkv,
                     scale * kLog2e, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* out, int T,
                               int W, int Hq, int Hkv, int d, int mode, float scale,
                               hipStream_t stream) {
  if (mode == 0) {
    if (d == 32) return launch<32, 0>(q, k, v, out, T, W, Hq, Hkv, scale, stream);
    if (d == 64) return launch<64, 0>(q, k, v, out, T, W, Hq, Hkv, scale, stream);
    return launch<128, 0>(q, k, v, out, T, W, Hq, Hkv, scale, stream);
  }
  if (d == 32) return launch<32, 1>(q, k, v, out, T, W, Hq, Hkv, scale, stream);
  if (d == 64) return launch<64, 1>(q, k, v, out, T, W, Hq, Hkv, scale, stream);
  return launch<128, 1>(q, k, v, out, T, W, Hq, Hkv, scale, stream);
}

}  // namespace swa
