// Banded sliding-window attention prefill for bfloat16 on gfx950 matrix cores.
//
// What is computed (robocikowo glossary "Sliding Window Attention", opening
// definition; Ultralytics glossary, section "Come cresce la finestra con la
// profondita"): out_i = softmax over the keys j of i's window of
// scale * q_i . k_j, applied to the v_j.  Causal window 0 <= i-j <= W-1,
// symmetric window |i-j| <= floor(W/2), both clipped to [0, T).
//
// Work decomposition: one workgroup = 128 query rows of one query head, four
// waves of 32 rows; two workgroups per CU at d = 128 (register-bound), three
// at d = 64, five at d = 32, so that the tile loads and barriers of one
// workgroup hide behind the work of the others.  (Softmax and matrix
// products overlap only within a wave, hence the mixed regions below.)
// Key/value tiles of 64 rows are visited only where they intersect the union
// of the block's windows, so the work is O(T * W * d) and no [T, T] matrix
// exists.
//
// Per tile:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16 with the K tile (LDS) as the A
//                 operand and the wave's Q rows (registers) as the B operand,
//                 so each lane owns one query row and row statistics need one
//                 exchange between lanes l and l^32.
//   softmax       fp32, scores kept raw: p = exp2(s*c - m*c) with
//                 c = scale*log2(e) folded into one FMA.  The reference
//                 maximum m is raised lazily, only when a probability against
//                 it reaches 2^28 (detected from the block's partial sums, so
//                 no per-score maximum is needed on the common path); the
//                 accumulators are then rescaled and the block recomputed.
//                 Larger-than-one probabilities cost no precision (bf16 and
//                 fp32 are relative-precision formats) and stay far from
//                 overflow.  The row sum adds the bf16-rounded probabilities
//                 the product uses (packed dot2).  The mask is applied only on
//                 tiles crossing a window edge or the end of the sequence.
//   O^T += V^T P^T  P (bf16, straight from the score registers) is the B
//                 operand; V^T comes from the natural [key][dim] LDS tile
//                 through the transposing LDS read (ds_read_b64_tr_b16).
// Tiles are double-buffered in LDS and filled by direct buffer-to-LDS loads
// (no register staging): the next tile's loads are in flight while the
// current one is consumed; one barrier per tile.  LDS rows are
// unpadded; their 16-byte chunks are XOR-swizzled by row so that the K reads,
// the transposing V reads and the tile stores are all free of bank conflicts.
//
// Grouped-query heads: query head h reads KV head h / (Hq / Hkv); workgroups
// are ordered so that the heads of one group and neighbouring query blocks
// land on the same XCD and share K/V through its L2.
//
// Chunked prefill (MODE 2) is the causal kernel in key coordinates relative
// to the chunk's first token at position p: key r >= 0 is chunk row r, key
// r < 0 is position p + r, read from ring slot (p + r) mod W (Ultralytics
// ring-buffer paragraph).  Tiles are aligned to the chunk start, so a tile is
// wholly ring or wholly chunk; the window mask adds p + r >= 0.
//
// Dilated windows (MODES 3 and 4; aivaro answer 629, section 4.2): key j is
// visible from query i when i - j is a multiple of the dilation d and
// (i - j) / d lies in the plain window.  Rows of different residues mod d
// never meet, so a workgroup takes the rows r, r + d, r + 2d, ... of one
// residue class as a sequence of its own (row stride d * D) and runs the
// plain causal or symmetric window on it.
//
// Global tokens (MODES 5 and 6; aivaro answer 629, section 4.3): every row
// also attends to the G global keys (those at or before it in the causal
// mode).  They are visited after the window's tiles, as extra tiles whose
// rows are gathered from the global positions; a global key already inside a
// row's window is masked there so that no key counts twice.  The global rows
// themselves attend to every key: the leading workgroups of the same launch
// compute their split-K partials (global_rows_unit below), and the decode
// kernels' merge writes them.

#include "swa_device.h"
#include "swa_launch.h"
#include "swa_tile_math.h"

namespace swa {
namespace {

// vector instructions interleaved with the matrix products of interior-tile
// regions A and B (spread evenly over the region's products): 80 measured
// 0.6-2% faster than 56 on the Mistral-7B prefill (two boxes, alternated
// builds; 64, 72 and 96 also tried)
constexpr int kValuA = 80;
constexpr int kValuB = 80;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;   // query rows per workgroup
constexpr int kBN = 64;            // key rows per tile
static_assert(kBM == tm::kBM && kBN == tm::kBN, "the tile arithmetic's block and tile sizes");
// A row's accumulators are rescaled only when one of its probabilities
// against the current reference maximum reaches 2^28 (a lane's partial block
// sum reaches 2^32): until then every product term stays far from overflow
// and the exponent headroom costs no precision (bf16 and fp32 keep their
// relative precision at any scale).
constexpr float kBigSum = 4294967296.0f;
constexpr float kNoMax = -1.0e30f;
constexpr int kBufferFlags = 0x00020000;  // raw 32-bit buffer access

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
struct Geo {
  static constexpr int ROWB = D * 2;              // bytes per K/V row in LDS
  static constexpr int TILEB = kBN * ROWB;        // bytes per tile
  static constexpr int KS = D / 16;               // k-steps of S = K Q^T
  static constexpr int MD = D / 32;               // 32-dim output blocks
  static constexpr int NLD = TILEB / (kThreads * 16);  // direct loads per thread per tile
};

// XOR swizzle of a row's 16-byte chunks (LDS: 64 banks of 4 bytes, i.e. 16
// chunk slots per 256 bytes).  Chosen per row length so that
//   * the K operand read (16 lanes, 16 consecutive rows, one logical chunk),
//   * the transposing V read (32 lanes, 4 consecutive rows x two 32-byte
//     chunk pairs) and
//   * the tile stores (16 lanes, consecutive chunks)
// each touch every bank slot at most once.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  if (D == 64) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  return (row >> 2) & 3;
}

// Occupancy target (waves per SIMD): d = 128 needs the registers of two
// waves; smaller heads fit more, which hides the tile-load latency of short
// windows.
template <int D>
constexpr int kWavesPerSimd = D == 128 ? 2 : (D == 64 ? 3 : 5);
// the global-key modes carry one more tile body; at d = 32 it needs the
// registers of four waves per SIMD rather than five
template <int D, int MODE>
constexpr int kWavesFor = MODE >= 5 && D == 32 ? 4 : kWavesPerSimd<D>;

// ---------------------------------------------------------------------------
// Rows of global tokens on the matrix cores (aivaro answer 629, section 4.3:
// a global token attends to every token).  One wave (a unit) takes 32 (global row,
// query head) pairs of one KV head and one split of kGRowKeys keys: the pairs'
// query rows are gathered as the B operand, 64-key K/V tiles are loaded into
// LDS, and scores, masking (key <= the row's last key: its own position when
// causal, T - 1 otherwise), an exact per-tile online softmax and O^T += V^T P^T
// follow the tiled kernel.  The unnormalised partial (acc, max in log2 units,
// sum) of each pair goes to the split-K workspace, merged afterwards by the
// decode kernels' merge pass.  The units run as the leading workgroups of the
// window pass's launch (two per workgroup, each in one half of its LDS), so
// that they overlap the window pass instead of following it.
// keys per split: 128 measured best at Longformer shapes (11.5 us; 256: 12.3,
// 512: 15.2 us, the merge then costing less)
constexpr int kGRowKeys = 128;

template <int D, int MODE>
__device__ __forceinline__ void global_rows_unit(const __bf16* __restrict__ q,
                                                 const __bf16* __restrict__ k,
                                                 const __bf16* __restrict__ v,
                                                 const int32_t* __restrict__ gpos,
                                                 float* __restrict__ ws_acc, float* __restrict__ ws_m,
                                                 float* __restrict__ ws_l, int T, int Hq, int Hkv,
                                                 int ngl, float c, uint32_t qsign, int S,
                                                 int n_pchunks, int unit, int lane, char* lds_k,
                                                 char* lds_v) {
  using Gm = Geo<D>;
  constexpr int ROWB = Gm::ROWB, KS = Gm::KS, MD = Gm::MD;
  constexpr int TILEB = kBN * ROWB;
  constexpr int NL = TILEB / (64 * 16);  // direct loads per lane per tile

  const int G = Hq / Hkv;
  const int n_pairs = ngl * G;
  int id = unit;
  const int split = id % S;
  id /= S;
  const int pc = id % n_pchunks;
  const int kvh = id / n_pchunks;
  const int half = lane >> 5;

  // this lane's row: pair pi = pc * 32 + lane % 32 (global row pi / G, query
  // head kvh * G + pi % G); positions outside [0, T) and pairs past the last
  // are rows without keys
  const int pi = pc * 32 + (lane & 31);
  int gp = -1, h = 0;
  if (pi < n_pairs) {
    gp = gpos[pi / G];
    h = kvh * G + pi % G;
    if (gp < 0 || gp >= T) gp = -1;
  }
  const int s0 = tm::grow_split_begin(split, kGRowKeys);
  const int s1 = tm::grow_split_end(split, kGRowKeys, T);
  const int lim = tm::grow_row_limit(MODE == 0, gp, T, s1);  // last key of the row
  // the wave stops after the last key any of its rows sees
  int wlim = lim;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wlim = max(wlim, __shfl_xor(wlim, off));

  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (gp >= 0) w = *reinterpret_cast<const uint4*>(q + ((size_t)h * T + gp) * D + ks * 16 + half * 8);
    w.x ^= qsign;
    w.y ^= qsign;
    w.z ^= qsign;
    w.w ^= qsign;
    qf[ks] = __builtin_bit_cast(bf16x8, w);
  }
  const __bf16* kh = k + (size_t)kvh * T * D;
  const __bf16* vh = v + (size_t)kvh * T * D;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)kh, 0, T * ROWB, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)vh, 0, T * ROWB, kBufferFlags);

  const int kr = lane & 31;
  const int kf = swz<D>(kr);
  const int tr_s = lane & 15, tr_g = lane >> 4;
  const int tr_row = 4 * (tr_g >> 1) + (tr_s >> 2);
  const int tr_c0 = 2 * (tr_g & 1) + ((tr_s & 3) >> 1);
  const int tr_flo = swz<D>(tr_row), tr_fhi = swz<D>(tr_row + 8);
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = f32x16{};
  float m = -INFINITY, l = 0.f;  // raw-score maximum and sum of this lane's row

  for (int k0 = s0; k0 <= wlim; k0 += kBN) {
    // the tile: rows past T re-read row T - 1 (finite, masked); the previous
    // tile's LDS reads are complete before it is overwritten
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int o16 = (64 * j + lane) * 16;
      const int row = o16 / ROWB;
      const int off = tm::grow_src_row(k0, row, T) * ROWB + ((((o16 % ROWB) / 16) ^ swz<D>(row)) * 16);
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass mishandles this builtin
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(lds_k + 64 * j * 16), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(lds_v + 64 * j * 16), 16, off, 0, 0, 0);
#else
      (void)rk, (void)rv, (void)off;
#endif
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tile is in LDS (one wave: no barrier)

    f32x16 sb[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sb[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds_k + (mb * 32 + kr) * ROWB + (((2 * ks + half) ^ kf) * 16));
        sb[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sb[mb], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (key > lim) sb[mb][r] = -INFINITY;
        mx = fmaxf(mx, sb[mb][r]);
      }
    }
    mx = max_lane_pair(mx);  // lanes l and l^32 hold the same row
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // a row without keys so far
    const float alpha = __builtin_amdgcn_exp2f((m - m_use) * c);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[md][r] *= alpha;
    }
    const float mc = -m_use * c;
    bf16x8 p[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sb[mb][8 * k2 + 2 * e], c, mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sb[mb][8 * k2 + 2 * e + 1], c, mc));
          w[e] = pack_bf16x2(p0, p1);
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]), ones, l, false);
        }
        p[2 * mb + k2] = __builtin_bit_cast(bf16x8, w);
      }
    }
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const int vlo = tr_row * ROWB + (((4 * md + tr_c0) ^ tr_flo) * 16) + (tr_s & 1) * 8;
      const int vhi = (tr_row + 8) * ROWB + (((4 * md + tr_c0) ^ tr_fhi) * 16) + (tr_s & 1) * 8;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const char* src = lds_v + kk * 16 * ROWB;
        const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + vlo));
        const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + vhi));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[kk], o[md], 0, 0, 0);
      }
    }
  }

  // ---- the pair's partial (the merge computes sum_s 2^(m_s - M) acc_s / ...)
  const float l_tot = l + __shfl_xor(l, 32);
  if (gp >= 0) {
    const size_t slot = ((size_t)kvh * n_pairs + pi) * S + split;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int dim = 32 * md + 8 * rq + 4 * half;
        *reinterpret_cast<float4*>(ws_acc + slot * D + dim) =
            make_float4(o[md][4 * rq], o[md][4 * rq + 1], o[md][4 * rq + 2], o[md][4 * rq + 3]);
      }
    }
    if (half == 0) {
      ws_m[slot] = m == -INFINITY ? -1.0e30f : m * c;
      ws_l[slot] = l_tot;
    }
  }
}

// MODE: 0 causal, 1 symmetric, 2 causal chunk continuing a ring cache (Tseq
// is then the chunk length; kring/vring/pos/hkv_seq are used by MODE 2 only),
// 3 causal dilated, 4 symmetric dilated (dil is used by MODES 3, 4, 7, 8),
// 5 causal and 6 symmetric window plus the ngl global keys at gpos (MODES 5
// to 8), 7 causal and 8 symmetric dilated window plus global keys.
template <int D, int MODE>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kWavesFor<D, MODE>, kWavesFor<D, MODE>)))
void prefill_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                         const __bf16* __restrict__ v, __bf16* __restrict__ out, int Tseq,
                         int W, int Hq, int Hkv, float c, uint32_t qsign, int n_qtiles,
                         const __bf16* __restrict__ kring, const __bf16* __restrict__ vring,
                         const int32_t* __restrict__ pos, int hkv_seq, int dil,
                         const int32_t* __restrict__ gpos, int ngl,
                         float* __restrict__ gr_acc, float* __restrict__ gr_m,
                         float* __restrict__ gr_l, int gr_S, int gr_pchunks, int gr_wgs) {
  constexpr bool kCausal = MODE != 1 && MODE != 4 && MODE != 6 && MODE != 8;
  constexpr bool kChunk = MODE == 2;
  constexpr bool kDil = MODE == 3 || MODE == 4 || MODE == 7 || MODE == 8;
  constexpr bool kGlobal = MODE >= 5;
  using Gm = Geo<D>;
  constexpr int ROWB = Gm::ROWB, TILEB = Gm::TILEB, KS = Gm::KS;
  constexpr int MD = Gm::MD, NLD = Gm::NLD;
  // two stages of K and V tiles, as separate objects so the compiler can tell
  // the stage being filled by direct loads from the stage being read
  __shared__ __attribute__((aligned(1024))) char lds_k0[TILEB];
  __shared__ __attribute__((aligned(1024))) char lds_v0[TILEB];
  __shared__ __attribute__((aligned(1024))) char lds_k1[TILEB];
  __shared__ __attribute__((aligned(1024))) char lds_v1[TILEB];
  // global modes: the positions of the global key tile held in each stage
  __shared__ __attribute__((aligned(16))) int lds_gp[2][kGlobal ? kBN : 1];

  // global modes: the first gr_wgs workgroups compute the global rows, two
  // units each (waves 0 and 1, each in its own LDS stage)
  if constexpr (kGlobal) {
    if ((int)blockIdx.x < gr_wgs) {
      const int w = threadIdx.x >> 6;
      const int unit = (int)tm::grow_unit(blockIdx.x, w);
      if (w < 2 && unit < Hkv * gr_pchunks * gr_S) {
        global_rows_unit<D, kCausal ? 0 : 1>(q, k, v, gpos, gr_acc, gr_m, gr_l, Tseq, Hq, Hkv, ngl,
                                             c, qsign, gr_S, gr_pchunks, unit, threadIdx.x & 63,
                                             w ? lds_k1 : lds_k0, w ? lds_v1 : lds_v0);
      }
      return;
    }
  }

  // ---- which (query head, query block) this workgroup owns
  const int G = Hq / Hkv;
  int id = (int)blockIdx.x - gr_wgs;
  const int nwg = (int)gridDim.x - gr_wgs;
  // consecutive ids go round-robin to the 8 XCDs: give each XCD a contiguous range
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int hg = id % G;
  const int rest = id / G;
  const int qt = rest % n_qtiles;
  int kvh = rest / n_qtiles;
  int cls = 0;  // dilated modes: the residue class of this workgroup's rows
  if constexpr (kDil) {
    cls = kvh % dil;
    kvh /= dil;
  }
  const int h = kvh * G + hg;
  // T rows of stride RS elements: the sequence itself, or one residue class
  const int T = kDil ? tm::class_rows(Tseq, cls, dil) : Tseq;
  const int RS = kDil ? dil * D : D;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + (lane & 31);  // the query row this lane owns

  const __bf16* qh = q + (size_t)h * Tseq * D + (size_t)cls * D;
  const __bf16* kh = k + (size_t)kvh * Tseq * D + (size_t)cls * D;
  const __bf16* vh = v + (size_t)kvh * Tseq * D + (size_t)cls * D;
  // global keys sit at sequence positions (outside any residue class)
  const __bf16* kg = k + (size_t)kvh * Tseq * D;
  const __bf16* vg = v + (size_t)kvh * Tseq * D;
  // a dilated class may be shorter than the longest one (or empty): a query
  // block past its end has nothing to do (uniform over the workgroup)
  if constexpr (kDil) {
    if (q0 >= T) return;
  }

  // chunk mode: position of the chunk's first token; the lowest key is -pstart
  int pstart = 0;
  if constexpr (kChunk) {
    pstart = pos[kvh / hkv_seq];
    if (pstart < 0) {  // inactive sequence: zero rows (uniform over the workgroup)
      if (qi < T) {
        __bf16* orow = out + ((size_t)h * Tseq + qi) * D;
#pragma unroll
        for (int md = 0; md < Gm::MD; ++md)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
            *reinterpret_cast<uint2*>(orow + 32 * md + 8 * rq + 4 * half) = make_uint2(0, 0);
      }
      return;
    }
  }

  const int hw = W >> 1;
  int lo, hi;
  if (kCausal) {
    lo = SWA_TM_CAUSAL_BLOCK_LO(q0, W, pstart);
    hi = SWA_TM_CAUSAL_BLOCK_HI(q0, T);
  } else {
    lo = SWA_TM_SYM_BLOCK_LO(q0, hw);
    hi = SWA_TM_SYM_BLOCK_HI(q0, T, hw);
  }
  int kt0;
  if constexpr (kChunk) {
    kt0 = tm::floor_tile(lo);  // floor division
  } else {
    kt0 = lo / kBN;
  }
  const int kt1 = hi / kBN;
  // global modes: the global key tiles follow the window's, as kt1+1 .. kt_end
  const int kt_end = kGlobal ? tm::global_tiles_end(kt1, ngl) : kt1;

  // this wave's rows and key range
  const bool wave_active = qw0 < T;
  const int qlast = SWA_TM_WAVE_LAST(qw0, T);
  const int wlo = SWA_TM_WAVE_LO(kCausal, qw0, W, hw, pstart);
  const int whi = SWA_TM_WAVE_HI(kCausal, qlast, T, hw);

  // ---- Q rows as B operands, zero beyond the sequence; a negative scale is
  // folded into Q's sign bits (exact) so that c > 0 below.
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (qi < T) w = *reinterpret_cast<const uint4*>(qh + (size_t)qi * RS + ks * 16 + half * 8);
    w.x ^= qsign;
    w.y ^= qsign;
    w.z ^= qsign;
    w.w ^= qsign;
    qf[ks] = __builtin_bit_cast(bf16x8, w);
  }

  // ---- global -> LDS tile copy with direct (buffer -> LDS) loads.  Load j
  // of this thread fills the 16 bytes at LDS offset (j*kThreads + tid)*16 of
  // the tile (each wave writes 1 KB contiguously) and fetches the logical
  // chunk the swizzle keeps there.  In the last, partial tile the rows past T
  // re-read row T-1, so every LDS row holds finite data (their scores are
  // masked to zero weight, and 0 * finite = 0 in the product).
  int src_off[NLD], src_row[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int o = tm::load_lds_offset(j, tid, kThreads);
    const int row = tm::load_row(o, ROWB);
    src_row[j] = row;
    src_off[j] = (tm::load_chunk(o, ROWB) ^ swz<D>(row)) * 16;
  }
  auto load_tile = [&](char* Kdst, char* Vdst, int kt) __attribute__((always_inline)) {
    const int kbase = kt * kBN;
    if constexpr (kGlobal) {
      if (kt > kt1) {
        // a global key tile: row j holds the key at gpos[t0 + j]; rows past
        // the last global key, and positions outside [0, T), re-read a valid
        // row (masked in global_tile)
        const int t0 = (kt - kt1 - 1) * kBN;
        // the tile's 64 global positions, for the mask (same stage discipline
        // as the K/V tiles: written after the barrier that frees the stage)
        if (tid < kBN) lds_gp[(kt - kt0) & 1][tid] = gpos[tm::global_index(t0, tid, ngl)];
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)kg, 0, Tseq * ROWB, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)vg, 0, Tseq * ROWB, kBufferFlags);
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
          const int wbase = (j * kThreads + wave * 64) * 16;
          const int gp = tm::global_src_row(gpos[tm::global_index(t0, src_row[j], ngl)], Tseq);
          const int off = gp * ROWB + src_off[j];
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass mishandles this builtin
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(Kdst + wbase), 16, off, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(Vdst + wbase), 16, off, 0, 0, 0);
#else
          (void)rk, (void)rv, (void)wbase, (void)off;
#endif
        }
        return;
      }
    }
    if constexpr (kChunk) {
      if (kbase < 0) {
        // a ring tile: key r = kbase + row is position pstart + r < pstart, in
        // slot (pstart + r) mod W.  Rows before position 0 (never in a window)
        // re-read position 0, which every sequence with pstart >= 1 has written.
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kring + (size_t)kvh * W * D), 0, W * ROWB, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vring + (size_t)kvh * W * D), 0, W * ROWB, kBufferFlags);
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
          const int wbase = (j * kThreads + wave * 64) * 16;
          const unsigned slot = tm::ring_slot(pstart, kbase, src_row[j], W);
          const int off = (int)slot * ROWB + src_off[j];
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass mishandles this builtin
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(Kdst + wbase), 16, off, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(Vdst + wbase), 16, off, 0, 0, 0);
#else
          (void)rk, (void)rv, (void)wbase, (void)off;
#endif
        }
        return;
      }
    }
    const int last = tm::tile_last(T, kt);  // last valid row of this tile
    const int RSB = RS * 2;                  // bytes between consecutive rows
    // the resource starts at the tile and ends after its last valid row
    // (at most 64 rows: the size stays far inside int32 at any T)
    const int bytes = tm::tile_bytes(last, RSB, ROWB);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kh + (size_t)kbase * RS), 0, bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vh + (size_t)kbase * RS), 0, bytes, kBufferFlags);
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int wbase = (j * kThreads + wave * 64) * 16;
      const int off = tm::tile_row_offset(src_row[j], last, RSB) + src_off[j];
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass mishandles this builtin
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(Kdst + wbase), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(Vdst + wbase), 16, off, 0, 0, 0);
#else
      (void)rk, (void)rv, (void)wbase, (void)off;
#endif
    }
  };

  // ---- per-lane LDS read offsets.
  // K (A operand of S^T): row mb*32 + lane%32, logical chunk 2*ks + half,
  // stored at chunk (2*ks + half) ^ f.
  const int kr = lane & 31;
  const int kf = swz<D>(kr);
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = kr * ROWB + (((2 * ks + half) ^ kf) * 16);
  // V (transposing read): source lane s of 16-lane group g addresses key row
  // 16*kk + 4*(g/2) + s/4 (plus 8 for the upper half) and dims
  // 32*md + 16*(g%2) + 4*(s%4), i.e. logical chunk 4*md + c0.  The two halves
  // sit 8 rows apart, which changes the swizzle, so each has its own offsets.
  const int tr_s = lane & 15, tr_g = lane >> 4;
  const int tr_row = 4 * (tr_g >> 1) + (tr_s >> 2);
  const int tr_c0 = 2 * (tr_g & 1) + ((tr_s & 3) >> 1);
  const int tr_flo = swz<D>(tr_row), tr_fhi = swz<D>(tr_row + 8);
  int voff_lo[MD], voff_hi[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) {
    voff_lo[md] = tr_row * ROWB + (((4 * md + tr_c0) ^ tr_flo) * 16) + (tr_s & 1) * 8;
    voff_hi[md] = (tr_row + 8) * ROWB + (((4 * md + tr_c0) ^ tr_fhi) * 16) + (tr_s & 1) * 8;
  }

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = f32x16{};
  // raw-score reference maximum of this lane's row; it starts so low that the
  // first visited keys raise it, yet -m_ref * c stays finite (c <= 1478 for
  // every scale the library accepts), so a masked score gives exp2(-inf) = 0
  float m_ref = kNoMax;
  float l_part = 0.f;    // this lane's share of the row sum
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // ---- tile building blocks
  auto kread = [&](const char* Ks, int mb, int ks) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(Ks + mb * 32 * ROWB + koff[ks]);
  };
  // O^T += V^T P^T for 16 keys (kk).  Element j of the P operand in lane l
  // holds key 16*kk + 8*(j/4) + 4*(l/32) + j%4.  The A operand must hold V at
  // those keys for dim 32*md + l%32; two transposing reads give exactly that:
  // within each 16-lane group, lane i receives component i%4 of the 8 bytes
  // addressed by lane 4*j + i/4, and each source lane addresses 4 consecutive
  // dims of one key row.
  auto vread = [&](const char* Vs, int md, int kk) __attribute__((always_inline)) -> bf16x8 {
    const char* src = Vs + kk * 16 * ROWB;
    const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + voff_lo[md]));
    const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + voff_hi[md]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // probabilities of one 32-key half against the current reference maximum,
  // packed as two bf16 B operands, with their (rounded) sum
  auto probs = [&](const f32x16& s, float mc, bf16x8* p, float& lsum) __attribute__((always_inline)) {
    lsum = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * k2 + 2 * e], c, mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * k2 + 2 * e + 1], c, mc));
        w[e] = pack_bf16x2(p0, p1);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]), ones, lsum, false);
      }
      p[k2] = __builtin_bit_cast(bf16x8, w);
    }
  };
  // When a block's probabilities grew too large for some row (partial sum
  // >= 2^32; also the first visited block, whose reference maximum is
  // -1e30), raise the reference maximum of every row whose block maximum
  // exceeds it and rescale the accumulators; the caller recomputes the block.
  // Returns true when anything was rescaled.
  auto raise_max = [&](const f32x16* sb, int nb, float lsum) __attribute__((always_inline)) -> bool {
    if (!__ballot(lsum >= kBigSum)) return false;
    float mx = -INFINITY;
    for (int b = 0; b < nb; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sb[b][r]);
    mx = max_lane_pair(mx);  // lanes l and l^32 hold the same row
    const bool grow = mx > m_ref;
    const float m_new = grow ? mx : m_ref;
    const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * c);
    m_ref = m_new;
    l_part *= alpha;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[md][r] *= alpha;
    }
    return true;
  };

  // opaque use: makes the speculative probabilities exist at this point, so
  // they are computed inside the overlap region rather than sunk into a branch
  auto pin = [&](bf16x8* p, float& l) __attribute__((always_inline)) {
    uint4 w0 = __builtin_bit_cast(uint4, p[0]), w1 = __builtin_bit_cast(uint4, p[1]);
#if defined(__HIP_DEVICE_COMPILE__)  // register constraints exist only for the GPU pass
    __asm__ volatile("" : "+v"(w0.x), "+v"(w0.y), "+v"(w0.z), "+v"(w0.w));
    __asm__ volatile("" : "+v"(w1.x), "+v"(w1.y), "+v"(w1.z), "+v"(w1.w), "+v"(l));
#endif
    p[0] = __builtin_bit_cast(bf16x8, w0);
    p[1] = __builtin_bit_cast(bf16x8, w1);
  };

  // symmetric windows: key k0 + kc (kc = 32 * mb + 8 * (r / 4) + 4 * half +
  // r % 4 for score register r of block mb) counts for this lane's row when
  // mlo <= kc - 4 * half <= mhi
  auto mask_block = [&](f32x16& sb, int mb, const tm::SymRange& mr) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kc = mb * 32 + 8 * (r >> 2) + (r & 3);
      if (!tm::sym_visible(mr, kc)) sb[r] = -INFINITY;
    }
  };

  // A tile inside every row's window.  Three regions, each mixing matrix and
  // vector work so that one wave keeps both busy:
  //   A: S of keys 32..63        | probabilities of keys 0..31
  //   B: O += V P for keys 0..31 | probabilities of keys 32..63
  //   C: O += V P for keys 32..63
  // Probabilities are computed against the current reference maximum; the
  // rare tile that raises it recomputes them after the rescale.  A wave in
  // regions A and B issues at raised priority, so on a SIMD shared by two
  // waves the one with vector work to interleave goes first and the other's
  // matrix-only work fills the gaps (measured about 1% faster than equal
  // priority).
  //
  // Masked (symmetric windows): a tile crossing a window edge or the sequence
  // end runs the same schedule, with a mask on each 32-key block that some
  // rows see only in part (bit b of the mask set: block b); key k0 + kc
  // counts for this lane's row when mlo <= kc - 4 * half <= mhi, tested on
  // the block's scores before their probabilities.
  auto interior_tile = [&](const char* Ks, const char* Vs, auto masked, tm::SymRange mr) __attribute__((always_inline)) {
    constexpr int kMask = decltype(masked)::value;
    // S for keys 0..31: all K operands requested up front
    bf16x8 ka[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = kread(Ks, 0, ks);
    f32x16 s0 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], s0, 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);
    __builtin_amdgcn_sched_barrier(0);

    // region A: S for keys 32..63 | probabilities of keys 0..31
    __builtin_amdgcn_s_setprio(3);
    bf16x8 p0[2], p1[2];
    float l0, l1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = kread(Ks, 1, ks);
    f32x16 s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], s1, 0, 0, 0);
    if constexpr ((kMask & 1) != 0) mask_block(s0, 0, mr);
    probs(s0, -m_ref * c, p0, l0);
    pin(p0, l0);
    __builtin_amdgcn_sched_group_barrier(0x100, KS / 2, 0);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuA / KS, 0);
      if (i < KS / 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (raise_max(&s0, 1, l0)) probs(s0, -m_ref * c, p0, l0);
    l_part += l0;

    // region B: O += V P for keys 0..31 | probabilities of keys 32..63
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(Vs, md, kk), p0[kk], o[md], 0, 0, 0);
    }
    if constexpr ((kMask & 2) != 0) mask_block(s1, 1, mr);
    probs(s1, -m_ref * c, p1, l1);
    pin(p1, l1);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * MD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuB / (2 * MD), 0);
      if (i < 2 * MD - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (raise_max(&s1, 1, l1)) probs(s1, -m_ref * c, p1, l1);
    l_part += l1;

    // region C: O += V P for keys 32..63
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(Vs, md, 2 + kk), p1[kk], o[md], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * MD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < 2 * MD - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // A symmetric tile of whose two 32-key blocks the wave's rows see only one
  // (block MB): that block alone, masked.
  auto block_tile = [&](const char* Ks, const char* Vs, auto mbc, tm::SymRange mr) __attribute__((always_inline)) {
    constexpr int MB = decltype(mbc)::value;
    f32x16 sb = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(Ks, MB, ks), qf[ks], sb, 0, 0, 0);
    mask_block(sb, MB, mr);
    bf16x8 pb[2];
    float lb;
    probs(sb, -m_ref * c, pb, lb);
    if (raise_max(&sb, 1, lb)) probs(sb, -m_ref * c, pb, lb);
    l_part += lb;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(Vs, md, 2 * MB + kk), pb[kk], o[md], 0, 0, 0);
    }
  };

  // A tile that crosses a window edge or the sequence end: mask, then the
  // same steps without overlap.
  auto edge_tile = [&](const char* Ks, const char* Vs, int k0) __attribute__((always_inline)) {
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(Ks, mb, ks), qf[ks], s[mb], 0, 0, 0);
    }
    if constexpr (kCausal && !kChunk) {
      // causal: window and sequence ends as one unsigned test per score,
      // 0 <= diff <= min(W - 1, qi) with diff = qi - key (keys >= 0; keys < T
      // follow for a row inside the sequence, and rows past T are never
      // stored)
      const unsigned span = tm::causal_edge_span(qi, W);
      const int d0 = qi - k0;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kc = mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);  // key - k0
          if (!tm::causal_edge_visible(d0, kc, span)) s[mb][r] = -INFINITY;
        }
      }
    } else {
      // symmetric and chunk modes: the single test keeps more values live
      // through the tile loop and spills there, so the bounds are tested
      // directly
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (!tm::edge_visible(kCausal, qi, key, T, W, pstart)) s[mb][r] = -INFINITY;
        }
      }
    }
    bf16x8 pb[4];
    float l0, l1;
    probs(s[0], -m_ref * c, pb, l0);
    probs(s[1], -m_ref * c, pb + 2, l1);
    if (raise_max(s, 2, fmaxf(l0, l1))) {
      probs(s[0], -m_ref * c, pb, l0);
      probs(s[1], -m_ref * c, pb + 2, l1);
    }
    l_part += l0 + l1;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(Vs, md, kk), pb[kk], o[md], 0, 0, 0);
    }
  };

  // A tile of gathered global keys (global modes): key t0 + kl sits at
  // gpos[t0 + kl] and counts for this row only when it is outside the row's
  // window (the window tiles already counted it) and, in the causal mode, not
  // after the row.  The lane's 32 keys are kl = 8 * g + 4 * half + e
  // (g = 0..7, e = 0..3), i.e. score register r of block mb holds key group
  // g = 4 * mb + r / 4; their verdicts are packed into one bit each first.
  // When at most 32 global keys are left, only the first 32-key block is
  // computed.
  auto global_tile = [&](const char* Ks, const char* Vs, int t0, const int* gp_tile) __attribute__((always_inline)) {
    // The global positions are the same for every row: when no row of the
    // wave has one of the tile's keys in its window (and, causal, none is
    // after a row), every valid key counts for every row and the per-key test
    // is skipped.  Lane j looks at key t0 + j of the tile.
    const int gl = gp_tile[lane];
    const bool gvalid = tm::global_valid(t0 + lane, gl, ngl, Tseq);
    int gmin = gvalid ? gl : 0x7fffffff, gmax = gvalid ? gl : -0x7fffffff - 1;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      gmin = ::min(gmin, __shfl_xor(gmin, off));
      gmax = ::max(gmax, __shfl_xor(gmax, off));
    }
    const int rlo = kDil ? cls + dil * qw0 : qw0;  // the wave's rows as sequence positions
    const int rhi = kDil ? cls + dil * qlast : qlast;
    const int wcls = tm::global_wave_class(kCausal, rlo, rhi, gmin, gmax, W, dil);
    uint32_t okbits = 0;
    if (wcls == tm::kGlobalAll) {
      okbits = tm::global_lane_bits(__ballot(gvalid), half);
    } else if (wcls == tm::kGlobalSome) {
      const int rpos = kDil ? cls + dil * qi : qi;  // this lane's row as a sequence position
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int4 gp4 = *reinterpret_cast<const int4*>(gp_tile + 8 * g + 4 * half);
        const int gpv[4] = {gp4.x, gp4.y, gp4.z, gp4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = t0 + 8 * g + 4 * half + e;
          const bool ok = tm::global_counts(kCausal, kDil, rpos, gpv[e], idx, ngl, Tseq, W, dil);
          okbits |= (uint32_t)ok << (4 * g + e);
        }
      }
    }
    // one 32-key block at a time, and only the blocks holding global keys
    const int nblk = ngl - t0 > 32 ? 2 : 1;
#pragma unroll 1
    for (int mb = 0; mb < nblk; ++mb) {
      f32x16 sb = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(Ks, mb, ks), qf[ks], sb, 0, 0, 0);
      const uint32_t bits = okbits >> (16 * mb);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (!((bits >> r) & 1u)) sb[r] = -INFINITY;
      }
      bf16x8 pb[2];
      float lb;
      probs(sb, -m_ref * c, pb, lb);
      if (raise_max(&sb, 1, lb)) probs(sb, -m_ref * c, pb, lb);
      l_part += lb;
#pragma unroll
      for (int md = 0; md < MD; ++md) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(Vs, md, 2 * mb + kk), pb[kk], o[md], 0, 0, 0);
      }
    }
  };

  // One tile: wait for its loads (issued during the previous tile) and for
  // every wave to be done with the other stage, refill that stage with the
  // next tile, then consume this one.
  auto step = [&](const char* Ks, const char* Vs, char* Kn, char* Vn, int kt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (kt < kt_end) load_tile(Kn, Vn, kt + 1);
    const int k0 = kt * kBN;
    if (!tm::tile_visited(wave_active, wlo, whi, k0)) return;
    const bool full = tm::tile_full(kCausal, kChunk, k0, qw0, qlast, T, W, pstart);
    if (full) {
      interior_tile(Ks, Vs, std::integral_constant<int, 0>{}, tm::SymRange{0, 0});
    } else if constexpr (!kCausal && !tm::sym_blocks_classified(D)) {
      // symmetric: keys k0 + kc with qi - hw <= k0 + kc <= min(qi + hw, T - 1)
      interior_tile(Ks, Vs, std::integral_constant<int, 3>{}, tm::sym_range(qi, k0, half, T, W));
    } else if constexpr (!kCausal) {
      // symmetric: keys k0 + kc with qi - hw <= k0 + kc <= min(qi + hw, T - 1);
      // each 32-key block is skipped, taken whole or masked, as the wave's
      // rows see it (the classes are uniform over the wave)
      const tm::SymRange mr = tm::sym_range(qi, k0, half, T, W);
      const int c0 = tm::sym_block_class(k0, qw0, qlast, T, W);
      const int c1 = tm::sym_block_class(k0 + 32, qw0, qlast, T, W);
      if (c1 == tm::kSymNone) {
        block_tile(Ks, Vs, std::integral_constant<int, 0>{}, mr);
      } else if (c0 == tm::kSymNone) {
        block_tile(Ks, Vs, std::integral_constant<int, 1>{}, mr);
      } else if (c0 == tm::kSymAll) {
        interior_tile(Ks, Vs, std::integral_constant<int, 2>{}, mr);
      } else if (c1 == tm::kSymAll) {
        interior_tile(Ks, Vs, std::integral_constant<int, 1>{}, mr);
      } else {
        interior_tile(Ks, Vs, std::integral_constant<int, 3>{}, mr);
      }
    } else {
      edge_tile(Ks, Vs, k0);
    }
  };
  load_tile(lds_k0, lds_v0, kt0);
  for (int kt = kt0; kt <= kt1; kt += 2) {
    step(lds_k0, lds_v0, lds_k1, lds_v1, kt);
    if (kt + 1 > kt1) break;
    step(lds_k1, lds_v1, lds_k0, lds_v0, kt + 1);
  }
  // global modes: the global key tiles, in a loop of their own (inside the
  // window loop their code would raise its register pressure); the last
  // window step already requested the first of them.  Tile kt sits in stage
  // (kt - kt0) & 1.
  if constexpr (kGlobal) {
    for (int kt = kt1 + 1; kt <= kt_end; ++kt) {
      const int st = (kt - kt0) & 1;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      if (kt < kt_end) load_tile(st ? lds_k0 : lds_k1, st ? lds_v0 : lds_v1, kt + 1);
      if (wave_active) global_tile(st ? lds_k1 : lds_k0, st ? lds_v1 : lds_v0, (kt - kt1 - 1) * kBN, lds_gp[st]);
    }
  }

  // ---- epilogue: divide by the row sum, round to bf16, store.  The
  // row-sum exchange involves both wave halves, so it precedes the guard.
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (qi < T) {
    const float inv = 1.0f / l_tot;
    __bf16* orow;
    if constexpr (kDil) {
      orow = out + (size_t)h * Tseq * D + (size_t)cls * D + (size_t)qi * RS;
    } else {
      orow = out + ((size_t)h * T + qi) * D;
    }
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

// ---------------------------------------------------------------------------
// Short windows.  When every window of 32 consecutive rows fits the 64 keys
// starting kOff keys before the first of them (causal W <= 33: kOff = 32;
// symmetric floor(W/2) <= 16: kOff = 16), one wave computes its 32 rows from
// one key block of its own: a workgroup is a single wave (no barriers, no
// idle waves), the softmax is exact in two passes over the block (maximum,
// then exponentials), and there is no online rescaling.  Same score layout,
// operand reads and LDS swizzle as the tiled kernel above.
template <int MODE>
constexpr int kShortOff = MODE == 0 ? 32 : 16;
// query heads of a KV group per short-window workgroup (at most): two
// measured best (TinyMistral 22.3 -> 20.2 us warm, 37 -> 33 us after a cache
// flush by writing; four: 20.6 / 32.5 us)
constexpr int kShortGroup = 2;

bool short_window(int W, int mode) { return mode == 0 ? W <= 33 : (W >> 1) <= 16; }

// The occupancy target keeps the matrix results in ordinary registers (with
// one wave per workgroup the compiler otherwise keeps them in accumulation
// registers and copies them out).
//
// NW > 1 (grouped query heads): a workgroup is NW waves, the same 32 rows of
// NW query heads of one KV group; the key block is loaded once into LDS, each
// wave issuing 1/NW of the direct loads, and one barrier makes it visible.
template <int D, int MODE, int NW = 1>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D>)))
void prefill_short_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ out, int T, int W, int Hq, int Hkv, float c, uint32_t qsign,
    int n_wtiles) {
  using Gm = Geo<D>;
  constexpr int ROWB = Gm::ROWB, KS = Gm::KS, MD = Gm::MD;
  constexpr int BLOCKB = 64 * ROWB;      // 64 key rows
  constexpr int NL = BLOCKB / (64 * 16);  // direct loads per lane per block (one wave)
  static_assert(NL % NW == 0, "the block's loads split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char lds_k[BLOCKB];
  __shared__ __attribute__((aligned(1024))) char lds_v[BLOCKB];

  const int G = Hq / Hkv;
  int id = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int ng = G / NW;  // workgroups per (KV head, row block)
  const int hg = (id % ng) * NW + (NW > 1 ? (int)(threadIdx.x >> 6) : 0);
  const int rest = id / ng;
  const int wt = rest % n_wtiles;
  const int kvh = rest / n_wtiles;
  const int h = kvh * G + hg;

  const int lane = threadIdx.x & 63;
  const int wave = NW > 1 ? (int)(threadIdx.x >> 6) : 0;
  const int half = lane >> 5;
  const int qw0 = wt * 32;
  const int qi = qw0 + (lane & 31);
  const int kb0 = qw0 - kShortOff<MODE>;  // key of LDS row 0 (may be negative)

  const __bf16* qh = q + (size_t)h * T * D;

  // ---- the key block, rows clamped into [0, T) (out-of-range rows hold
  // finite data and are masked below); load j of a lane fills LDS bytes
  // [(64*j + lane)*16, +16).  The resource starts at the block's first row
  // inside the sequence (blo) and covers at most its 64 rows, so offsets stay
  // small at any T.
  {
    const tm::ShortBlock sbk = tm::short_block(qw0, kShortOff<MODE>, T);
    const int blo = sbk.blo;
    const int bhi = sbk.bhi;
    const __bf16* kblk = k + ((size_t)kvh * T + blo) * D;
    const __bf16* vblk = v + ((size_t)kvh * T + blo) * D;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)kblk, 0, (bhi - blo + 1) * ROWB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)vblk, 0, (bhi - blo + 1) * ROWB, kBufferFlags);
#pragma unroll
    for (int jj = 0; jj < NL / NW; ++jj) {
      const int j = wave * (NL / NW) + jj;
      const int o = (64 * j + lane) * 16;
      const int row = o / ROWB;
      const int src = tm::short_src_row(sbk, row);
      const int off = (src - blo) * ROWB + ((((o % ROWB) / 16) ^ swz<D>(row)) * 16);
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass mishandles this builtin
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(lds_k + 64 * j * 16), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(lds_v + 64 * j * 16), 16, off, 0, 0, 0);
#else
      (void)rk, (void)rv, (void)off;
#endif
    }
  }
  // ---- Q rows as B operands (sign of a negative scale folded in)
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 r = make_uint4(0, 0, 0, 0);
    if (qi < T) r = *reinterpret_cast<const uint4*>(qh + (size_t)qi * D + ks * 16 + half * 8);
    r.x ^= qsign;
    r.y ^= qsign;
    r.z ^= qsign;
    r.w ^= qsign;
    qf[ks] = __builtin_bit_cast(bf16x8, r);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's part of the block is in LDS
  if constexpr (NW > 1) __syncthreads();  // and every other wave's part

  // ---- S^T = K Q^T for the 64 keys (two 32-key blocks), masked
  const int kr = lane & 31;
  const int kf = swz<D>(kr);
  f32x16 s[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    s[mb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(
          lds_k + (mb * 32 + kr) * ROWB + (((2 * ks + half) ^ kf) * 16));
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mb], 0, 0, 0);
    }
  }
  // The window and the sequence ends as one unsigned range test per score on
  // diff = qi - key, with the lane's bounds computed once: keys >= 0 means
  // diff <= qi; keys < T means diff > qi - T (automatic in the causal mode for
  // a row inside the sequence; rows past T are never stored).  A symmetric
  // row far past T gets dlo > dhi: the span wraps and keeps every score of its
  // clamped, finite rows.
  const tm::ShortMask smk = tm::short_mask(MODE == 0, qi, kb0, T, W);
  float mx = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kc = mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);  // key - kb0
      if (!tm::short_visible(smk, kc)) s[mb][r] = -INFINITY;
      mx = fmaxf(mx, s[mb][r]);
    }
  }
  mx = max_lane_pair(mx);  // lanes l and l^32 hold the same row
  // a row past T has no valid key: keep its (unstored) arithmetic finite
  if (mx == -INFINITY) mx = 0.f;

  // ---- probabilities (bf16, as the product uses them) and their sum
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  const float mc = -mx * c;
  bf16x8 p[4];
  float l = 0.f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[mb][8 * k2 + 2 * e], c, mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[mb][8 * k2 + 2 * e + 1], c, mc));
        w[e] = pack_bf16x2(p0, p1);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]), ones, l, false);
      }
      p[2 * mb + k2] = __builtin_bit_cast(bf16x8, w);
    }
  }
  l += __shfl_xor(l, 32);

  // ---- O^T = V^T P^T over the 64 keys (transposing LDS reads, as above)
  const int tr_s = lane & 15, tr_g = lane >> 4;
  const int tr_row = 4 * (tr_g >> 1) + (tr_s >> 2);
  const int tr_c0 = 2 * (tr_g & 1) + ((tr_s & 3) >> 1);
  const int tr_flo = swz<D>(tr_row), tr_fhi = swz<D>(tr_row + 8);
  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) {
    o[md] = f32x16{};
    const int vlo = tr_row * ROWB + (((4 * md + tr_c0) ^ tr_flo) * 16) + (tr_s & 1) * 8;
    const int vhi = (tr_row + 8) * ROWB + (((4 * md + tr_c0) ^ tr_fhi) * 16) + (tr_s & 1) * 8;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const char* src = lds_v + kk * 16 * ROWB;
      const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + vlo));
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + vhi));
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[kk], o[md], 0, 0, 0);
    }
  }

  // ---- divide by the row sum, round to bf16, store
  if (qi < T) {
    const float inv = 1.0f / l;
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
hipError_t launch_short(const void* q, const void* k, const void* v, void* out, int T, int W,
                        int Hq, int Hkv, float c, uint32_t qsign, hipStream_t stream) {
  const int n_wtiles = (T + 31) / 32;
  const int G = Hq / Hkv;
#define SWA_SHORT(NW)                                                                              \
  hipLaunchKernelGGL((prefill_short_kernel<D, MODE, NW>), dim3((unsigned)((long long)n_wtiles * (Hq / NW))), \
                     dim3(64 * NW), 0, stream, static_cast<const __bf16*>(q),                     \
                     static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),                 \
                     static_cast<__bf16*>(out), T, W, Hq, Hkv, c, qsign, n_wtiles)
  // query heads of a KV group share the key block where the group allows
  if constexpr (kShortGroup >= 4) {
    if (G % 4 == 0) {
      SWA_SHORT(4);
      return hipGetLastError();
    }
  }
  if constexpr (kShortGroup >= 2) {
    if (G % 2 == 0) {
      SWA_SHORT(2);
      return hipGetLastError();
    }
  }
  SWA_SHORT(1);
#undef SWA_SHORT
  return hipGetLastError();
}

// softmax constant c = scale * log2(e) > 0; a negative scale is folded into
// Q's sign bits (bf16 negation is exact); scale 0 makes every weight equal
// while masked logits stay at -inf
void fold_scale(float scale, float& c, uint32_t& qsign) {
  c = scale * kLog2e;
  qsign = 0;
  if (c < 0.f) {
    c = -c;
    qsign = 0x80008000u;
  }
  if (c == 0.f) c = 1.0e-30f;
}

template <int D, int MODE>
hipError_t launch(const void* q, const void* k, const void* v, void* out, int T, int W, int Hq,
                  int Hkv, float scale, hipStream_t stream) {
  const int n_qtiles = (T + kBM - 1) / kBM;
  const long long nwg = (long long)n_qtiles * Hq;
  float c;
  uint32_t qsign;
  fold_scale(scale, c, qsign);
  if (short_window(W, MODE)) return launch_short<D, MODE>(q, k, v, out, T, W, Hq, Hkv, c, qsign, stream);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, MODE>), dim3((unsigned)nwg), dim3(kThreads), 0,
                     stream, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), static_cast<__bf16*>(out), T, W, Hq, Hkv, c,
                     qsign, n_qtiles, static_cast<const __bf16*>(nullptr),
                     static_cast<const __bf16*>(nullptr), static_cast<const int32_t*>(nullptr), 1,
                     1, static_cast<const int32_t*>(nullptr), 0, nullptr, nullptr, nullptr, 1, 1, 0);
  return hipGetLastError();
}

// Dilated windows: one workgroup per (query head, residue class, query block
// of the class's rows); the longest class has ceil(T / dil) rows.
// The global-row units of a global-key launch: split-K over kGRowKeys-key
// chunks of every (KV head, chunk of 32 (global row, query head) pairs); two
// units per workgroup, a multiple of 8 workgroups so that the window
// workgroups keep their XCD placement.  Workspace layout: acc, then the
// maxima, then the sums, as the merge reads them.
struct GlobalRows {
  float *acc, *m, *l;
  int S, pchunks, wgs;
};
GlobalRows global_rows_plan(float* ws, int T, int Hq, int Hkv, int ngl, int D) {
  GlobalRows g;
  g.S = (T + kGRowKeys - 1) / kGRowKeys;
  g.pchunks = (ngl * (Hq / Hkv) + 31) / 32;
  g.wgs = ngl > 0 ? (int)tm::grow_workgroups((long long)Hkv * g.pchunks * g.S) : 0;
  const size_t rows = (size_t)ngl * Hq * g.S;
  g.acc = ws;
  g.m = ws ? ws + rows * D : nullptr;
  g.l = ws ? g.m + rows : nullptr;
  return g;
}

template <int D, int MODE>
hipError_t launch_dilated(const void* q, const void* k, const void* v, void* out, int T, int W,
                          int Hq, int Hkv, float scale, int dil, hipStream_t stream,
                          const int32_t* gpos = nullptr, int ngl = 0, float* ws = nullptr) {
  const int n_qtiles = ((T + dil - 1) / dil + kBM - 1) / kBM;
  const GlobalRows gr = global_rows_plan(ws, T, Hq, Hkv, gpos ? ngl : 0, D);
  const long long nwg = (long long)n_qtiles * Hq * dil + gr.wgs;
  float c;
  uint32_t qsign;
  fold_scale(scale, c, qsign);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, MODE>), dim3((unsigned)nwg), dim3(kThreads), 0,
                     stream, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), static_cast<__bf16*>(out), T, W, Hq, Hkv, c,
                     qsign, n_qtiles, static_cast<const __bf16*>(nullptr),
                     static_cast<const __bf16*>(nullptr), static_cast<const int32_t*>(nullptr), 1,
                     dil, gpos, ngl, gr.acc, gr.m, gr.l, gr.S, gr.pchunks, gr.wgs);
  return hipGetLastError();
}

// Window plus global keys, with the global rows' split-K partials computed in
// the same launch (the merge writes those rows afterwards).
template <int D, int MODE>
hipError_t launch_global(const void* q, const void* k, const void* v, void* out, int T, int W,
                         int Hq, int Hkv, float scale, const int32_t* gpos, int ngl, float* ws,
                         hipStream_t stream) {
  const int n_qtiles = (T + kBM - 1) / kBM;
  const GlobalRows gr = global_rows_plan(ws, T, Hq, Hkv, ngl, D);
  const long long nwg = (long long)n_qtiles * Hq + gr.wgs;
  float c;
  uint32_t qsign;
  fold_scale(scale, c, qsign);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, MODE>), dim3((unsigned)nwg), dim3(kThreads), 0,
                     stream, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), static_cast<__bf16*>(out), T, W, Hq, Hkv, c,
                     qsign, n_qtiles, static_cast<const __bf16*>(nullptr),
                     static_cast<const __bf16*>(nullptr), static_cast<const int32_t*>(nullptr), 1,
                     1, gpos, ngl, gr.acc, gr.m, gr.l, gr.S, gr.pchunks, gr.wgs);
  return hipGetLastError();
}

// Chunked prefill: B sequences of n new tokens; heads are folded with the
// batch (B*Hq query heads, B*Hkv KV heads, ring heads likewise), and the
// kernel recovers the sequence of KV head kvh as kvh / Hkv.
template <int D>
hipError_t launch_chunk(const void* q, const void* k, const void* v, const void* k_ring,
                        const void* v_ring, const int32_t* pos, void* out, int B, int n, int W,
                        int Hq, int Hkv, float scale, hipStream_t stream) {
  const int n_qtiles = (n + kBM - 1) / kBM;
  const long long nwg = (long long)n_qtiles * Hq * B;
  float c;
  uint32_t qsign;
  fold_scale(scale, c, qsign);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, 2>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), static_cast<__bf16*>(out), n, W, Hq * B,
                     Hkv * B, c, qsign, n_qtiles, static_cast<const __bf16*>(k_ring),
                     static_cast<const __bf16*>(v_ring), pos, Hkv, 1,
                     static_cast<const int32_t*>(nullptr), 0, nullptr, nullptr, nullptr, 1, 1, 0);
  return hipGetLastError();
}

}  // namespace

int global_rows_mfma_splits(int T) { return (T + kGRowKeys - 1) / kGRowKeys; }

hipError_t launch_prefill_chunk_bf16(const void* q, const void* k, const void* v,
                                     const void* k_ring, const void* v_ring, const int32_t* pos,
                                     void* out, int B, int n, int W, int Hq, int Hkv, int d,
                                     float scale, hipStream_t stream) {
  if (d == 32) return launch_chunk<32>(q, k, v, k_ring, v_ring, pos, out, B, n, W, Hq, Hkv, scale, stream);
  if (d == 64) return launch_chunk<64>(q, k, v, k_ring, v_ring, pos, out, B, n, W, Hq, Hkv, scale, stream);
  return launch_chunk<128>(q, k, v, k_ring, v_ring, pos, out, B, n, W, Hq, Hkv, scale, stream);
}

hipError_t launch_prefill_global_window_bf16(const void* q, const void* k, const void* v,
                                             void* out, int T, int W, int Hq, int Hkv, int d,
                                             int mode, float scale, const int32_t* gpos, int ngl,
                                             int dil, float* ws, hipStream_t stream) {
  if (dil > 1) {  // dilated window plus global keys
    if (mode == 0) {
      if (d == 32) return launch_dilated<32, 7>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl, ws);
      if (d == 64) return launch_dilated<64, 7>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl, ws);
      return launch_dilated<128, 7>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl, ws);
    }
    if (d == 32) return launch_dilated<32, 8>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl, ws);
    if (d == 64) return launch_dilated<64, 8>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl, ws);
    return launch_dilated<128, 8>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl, ws);
  }
  if (mode == 0) {
    if (d == 32) return launch_global<32, 5>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, ws, stream);
    if (d == 64) return launch_global<64, 5>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, ws, stream);
    return launch_global<128, 5>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, ws, stream);
  }
  if (d == 32) return launch_global<32, 6>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, ws, stream);
  if (d == 64) return launch_global<64, 6>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, ws, stream);
  return launch_global<128, 6>(q, k, v, out, T, W, Hq, Hkv, scale, gpos, ngl, ws, stream);
}

hipError_t launch_prefill_dilated_bf16(const void* q, const void* k, const void* v, void* out,
                                       int T, int W, int Hq, int Hkv, int d, int mode,
                                       float scale, int dil, hipStream_t stream) {
  if (dil == 1) return launch_prefill_bf16(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, stream);
  if (mode == 0) {
    if (d == 32) return launch_dilated<32, 3>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
    if (d == 64) return launch_dilated<64, 3>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
    return launch_dilated<128, 3>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
  }
  if (d == 32) return launch_dilated<32, 4>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
  if (d == 64) return launch_dilated<64, 4>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
  return launch_dilated<128, 4>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
}

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
