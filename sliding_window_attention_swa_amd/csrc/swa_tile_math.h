// Index arithmetic of the bf16 prefill kernels: which key tiles a block of
// query rows visits, which keys each row counts, and where every tile load
// reads from.  The kernels call these functions, and a CPU program built
// from this same header (tests/tile_walk.cpp) walks the kernels' loops with
// them to check, shape by shape, that every load stays inside its buffer and
// that each row counts exactly the keys of its window (compared with the
// masks of the fp64 oracle).  Plain integer C++: no HIP types.
//
// Windows (robocikowo glossary "Sliding Window Attention", opening
// definition; Ultralytics glossary, section "Come cresce la finestra con la
// profondita"): causal keys i-W+1 .. i, symmetric keys i-W/2 .. i+W/2, both
// clipped to the sequence.  Ring slots follow the Ultralytics ring-buffer
// paragraph (position p in slot p mod W).
#pragma once

#if defined(__HIPCC__)
#define SWA_HD __host__ __device__ __forceinline__
#else
#define SWA_HD inline
#endif

namespace swa {
namespace tm {

constexpr int kBN = 64;   // keys per tile
constexpr int kBM = 128;  // query rows per block of the tiled kernel

#if defined(__HIP_DEVICE_COMPILE__)
SWA_HD int imin(int a, int b) { return ::min(a, b); }
SWA_HD int imax(int a, int b) { return ::max(a, b); }
#else
SWA_HD int imin(int a, int b) { return a < b ? a : b; }
SWA_HD int imax(int a, int b) { return a > b ? a : b; }
#endif

// ---------------------------------------------------------------- tiled kernel

// Rows of a dilated residue class: class cls (< dil) of a sequence of Tseq
// rows holds the rows cls, cls + dil, ...; its length.
SWA_HD int class_rows(int Tseq, int cls, int dil) { return (Tseq - cls + dil - 1) / dil; }

// The keys [lo, hi] the rows [q0, q0 + kBM - 1] of a block see (keys start at
// -pstart in the chunk mode, where key r is position pstart + r; pstart = 0
// otherwise), and the first tile holding them (floor division: chunk keys
// below 0 are ring positions); the last tile is hi / kBN.  The bounds are
// macros: as functions they perturb the compiler's instruction schedule of
// the kernels (same results, more registers).
#define SWA_TM_CAUSAL_BLOCK_LO(q0, W, pstart) ::swa::tm::imax(-(pstart), (q0) - (W) + 1)
#define SWA_TM_CAUSAL_BLOCK_HI(q0, T) ::swa::tm::imin((T) - 1, (q0) + ::swa::tm::kBM - 1)
#define SWA_TM_SYM_BLOCK_LO(q0, hw) ::swa::tm::imax(0, (q0) - (hw))
#define SWA_TM_SYM_BLOCK_HI(q0, T, hw) ::swa::tm::imin((T) - 1, (q0) + ::swa::tm::kBM - 1 + (hw))
SWA_HD int floor_tile(int key) { return key >= 0 ? key / kBN : -((kBN - 1 - key) / kBN); }

// Global modes: the global key tiles follow the window's, as kt1 + 1 .. end.
SWA_HD int global_tiles_end(int kt1, int ngl) { return kt1 + (ngl + kBN - 1) / kBN; }

// The 32 rows [qw0, qlast] of a wave and the keys [wlo, whi] any of them
// sees (macros, as above).
#define SWA_TM_WAVE_LAST(qw0, T) ::swa::tm::imin((qw0) + 31, (T) - 1)
#define SWA_TM_WAVE_LO(causal, qw0, W, hw, pstart) \
  ((causal) ? ::swa::tm::imax(-(pstart), (qw0) - (W) + 1) : ::swa::tm::imax(0, (qw0) - (hw)))
#define SWA_TM_WAVE_HI(causal, qlast, T, hw) \
  ((causal) ? (qlast) : ::swa::tm::imin((T) - 1, (qlast) + (hw)))

// Does the wave take part in tile k0 (its keys meet [wlo, whi])?
SWA_HD bool tile_visited(bool active, int wlo, int whi, int k0) {
  return active && k0 <= whi && k0 + kBN - 1 >= wlo;
}

// Does every row of the wave see every key of tile k0 (no mask needed)?
SWA_HD bool tile_full(bool causal, bool chunk, int k0, int qw0, int qlast, int T, int W,
                      int pstart) {
  const int hw = W >> 1;
  bool full;
  if (causal) {
    full = (k0 + kBN - 1 <= qw0) && (k0 >= qlast - W + 1) && (k0 + kBN <= T);
    if (chunk) full = full && k0 >= -pstart;
  } else {
    full = (k0 >= qlast - hw) && (k0 + kBN - 1 <= qw0 + hw) && (k0 + kBN <= T);
  }
  return full;
}

// Causal edge tile (not chunk): key k0 + kc counts for row qi when
// 0 <= qi - key <= min(W - 1, qi), as one unsigned test (keys >= 0 is
// diff <= qi; keys < T follow for a row inside the sequence).
SWA_HD unsigned causal_edge_span(int qi, int W) { return (unsigned)imin(W - 1, qi); }
SWA_HD bool causal_edge_visible(int d0, int kc, unsigned span) {
  return (unsigned)(d0 - kc) <= span;
}

// Edge tile, the bounds tested directly (the chunk mode): key counts for
// row qi when it is inside the sequence (< T) and the window (causal: not
// before the sequence's first position, -pstart).
SWA_HD bool edge_visible(bool causal, int qi, int key, int T, int W, int pstart) {
  const int hw = W >> 1;
  const int diff = qi - key;
  bool ok = key < T;
  if (causal) {
    ok = ok && diff >= 0 && diff < W && key >= -pstart;
  } else {
    ok = ok && diff >= -hw && diff <= hw;
  }
  return ok;
}

// Symmetric tile that some rows see only in part: key k0 + kc + 4 * half
// (kc = 32 * mb + 8 * (r / 4) + r % 4 for score register r of block mb)
// counts for row qi when mlo <= kc <= mhi.
struct SymRange {
  int mlo, mhi;
};
SWA_HD SymRange sym_range(int qi, int k0, int half, int T, int W) {
  const int hw = W >> 1;
  SymRange m;
  m.mlo = qi - hw - k0 - 4 * half;
  m.mhi = imin(qi + hw, T - 1) - k0 - 4 * half;
  return m;
}
SWA_HD bool sym_visible(const SymRange& m, int kc) { return !(kc < m.mlo || kc > m.mhi); }

// Symmetric windows: how the wave's rows [qw0, qlast] see the 32-key block
// starting at key kb.  kSymNone: no row sees any of its keys (the block is
// skipped); kSymAll: every row sees every key, all inside the sequence (no
// mask); kSymSome: anything else (masked per score).
// The kernels classify blocks at head sizes of 64 and more; at 32 the extra
// tile variants exceed the register budget of five waves per SIMD, and both
// blocks of an edge tile are masked.
constexpr int kSymNone = 0, kSymSome = 1, kSymAll = 2;
constexpr bool sym_blocks_classified(int D) { return D >= 64; }
SWA_HD int sym_block_class(int kb, int qw0, int qlast, int T, int W) {
  const int hw = W >> 1;
  if (kb + 31 < imax(0, qw0 - hw) || kb > imin(T - 1, qlast + hw)) return kSymNone;
  if (kb >= qlast - hw && kb + 31 <= qw0 + hw && kb + 32 <= T) return kSymAll;
  return kSymSome;
}

// Window tile kt of a sequence (or residue class) of T rows, RSB bytes from
// one row to the next and ROWB bytes per row: the buffer resource starts at
// the tile's first row and ends after its last valid row (at most 64 rows);
// LDS row `row` of the tile reads row min(row, last) (rows past the end
// re-read the last row: finite data, masked).
SWA_HD int tile_last(int T, int kt) { return T - 1 - kt * kBN; }
SWA_HD int tile_bytes(int last, int RSB, int ROWB) { return imin(last, kBN - 1) * RSB + ROWB; }
SWA_HD int tile_row_offset(int row, int last, int RSB) { return imin(row, last) * RSB; }

// Chunk mode, ring tile (kbase < 0): key kbase + row is position
// pstart + kbase + row, in slot (position) mod W; rows before position 0
// (never in a window) re-read position 0.
SWA_HD unsigned ring_slot(int pstart, int kbase, int row, int W) {
  return (unsigned)imax(pstart + kbase + row, 0) % (unsigned)W;
}

// Global modes: row `row` of global tile t0 holds the key at gpos[t0 + row];
// rows past the last global key, and positions outside [0, Tseq), re-read a
// valid row (masked by global_counts).
SWA_HD int global_index(int t0, int row, int ngl) { return imin(t0 + row, ngl - 1); }
SWA_HD int global_src_row(int gp, int Tseq) { return imin(imax(gp, 0), Tseq - 1); }

// Does global key number idx, at position gp, count for the row at sequence
// position rpos?  Only outside the row's (dilated) window, which already
// counted it, and not after the row when causal.
SWA_HD bool global_counts(bool causal, bool dilated, int rpos, int gp, int idx, int ngl, int Tseq,
                          int W, int dil) {
  const int hw = W >> 1;
  const int diff = rpos - gp;
  bool in_window;
  if (dilated) {  // on the row's grid, within the window's offsets
    const int m = diff / dil;
    in_window = diff == m * dil && (causal ? (m >= 0 && m < W) : (m >= -hw && m <= hw));
  } else {
    in_window = causal ? (diff >= 0 && diff < W) : (diff >= -hw && diff <= hw);
  }
  bool ok = idx < ngl && gp >= 0 && gp < Tseq && !in_window;
  if (causal) ok = ok && diff >= 0;
  return ok;
}

// Global key idx of a tile (at position gp) exists: idx < ngl, gp in [0, Tseq).
SWA_HD bool global_valid(int idx, int gp, int ngl, int Tseq) { return idx < ngl && gp >= 0 && gp < Tseq; }

// A wave's rows at sequence positions [rlo, rhi] (one dilation grid when
// dilated) against a tile's valid global keys at positions [gmin, gmax]
// (gmin > gmax: none).  kGlobalAll: no row has any of them in its window and
// none is after a causal row, so every valid key counts for every row;
// kGlobalNone: none counts (causal: all after every row); kGlobalSome: test
// each key with global_counts.
constexpr int kGlobalSome = 0, kGlobalAll = 1, kGlobalNone = 2;
SWA_HD int global_wave_class(bool causal, int rlo, int rhi, int gmin, int gmax, int W, int dil) {
  if (gmin > gmax) return kGlobalNone;
  if (causal) {
    if (gmin > rhi) return kGlobalNone;
    if ((long long)gmax < (long long)rlo - (long long)(W - 1) * dil) return kGlobalAll;
  } else {
    const long long reach = (long long)(W >> 1) * dil;
    if ((long long)gmax < rlo - reach || (long long)gmin > rhi + reach) return kGlobalAll;
  }
  return kGlobalSome;
}

// The lane's 32 key bits (bit 4g + e: key 8g + 4 half + e of the tile) from
// a mask with bit j for key j of the tile.
SWA_HD unsigned global_lane_bits(unsigned long long m, int half) {
  unsigned b = 0;
  for (int g = 0; g < 8; ++g) b |= (unsigned)((m >> (8 * g + 4 * half)) & 0xFull) << (4 * g);
  return b;
}

// LDS placement of a tile load: load j of thread tid fills the 16 bytes at
// (j * threads + tid) * 16 of the tile; it reads LDS row `row` of the tile,
// logical 16-byte chunk `chunk` of that row.
SWA_HD int load_lds_offset(int j, int tid, int threads) { return (j * threads + tid) * 16; }
SWA_HD int load_row(int lds_off, int ROWB) { return lds_off / ROWB; }
SWA_HD int load_chunk(int lds_off, int ROWB) { return (lds_off % ROWB) / 16; }

// ---------------------------------------------------------------- short windows

// The short-window kernel gives the 32 rows from qw0 the 64 keys from
// kb0 = qw0 - off (off = 32 causal, 16 symmetric); the resource covers the
// rows [blo, bhi] of the block inside the sequence and LDS row `row` reads
// row clamp(kb0 + row) of them.
struct ShortBlock {
  int kb0, blo, bhi;
};
SWA_HD ShortBlock short_block(int qw0, int off, int T) {
  ShortBlock b;
  b.kb0 = qw0 - off;
  b.blo = imax(b.kb0, 0);
  b.bhi = imin(b.kb0 + 63, T - 1);
  return b;
}
SWA_HD int short_src_row(const ShortBlock& b, int row) { return imin(imax(b.kb0 + row, b.blo), b.bhi); }

// Its window test: on diff = qi - key with the lane's bounds [dlo, dhi] as one
// unsigned test (keys >= 0 is diff <= qi; keys < T is diff > qi - T).
struct ShortMask {
  int d0;
  unsigned span;
};
SWA_HD ShortMask short_mask(bool causal, int qi, int kb0, int T, int W) {
  const int hw = W >> 1;
  const int dlo = causal ? 0 : imax(-hw, qi - T + 1);
  const int dhi = causal ? imin(W - 1, qi) : imin(hw, qi);
  ShortMask m;
  m.span = (unsigned)(dhi - dlo);
  m.d0 = qi - kb0 - dlo;
  return m;
}
SWA_HD bool short_visible(const ShortMask& m, int kc) { return (unsigned)(m.d0 - kc) <= m.span; }

// ---------------------------------------------------------------- global rows

// The global-rows kernel: split `split` of keys_per_split keys; the lane's
// row (global position gp, -1 for none) counts the keys up to lim; the wave
// visits the tiles k0 = s0, s0 + 64, ... up to the largest lim of its rows;
// LDS row `row` of tile k0 reads key min(k0 + row, T - 1).
SWA_HD int grow_split_begin(int split, int keys_per_split) { return split * keys_per_split; }
SWA_HD int grow_split_end(int split, int keys_per_split, int T) {
  return imin(T, split * keys_per_split + keys_per_split);
}
SWA_HD int grow_row_limit(bool causal, int gp, int T, int s1) {
  return gp < 0 ? -1 : imin(causal ? gp : T - 1, s1 - 1);
}
SWA_HD int grow_src_row(int k0, int row, int T) { return imin(k0 + row, T - 1); }
// The units run as the leading workgroups of the window launch, two per
// workgroup (waves 0 and 1): unit 2 * wg + wave, if below the unit count; the
// number of such workgroups is rounded up to a multiple of 8 so that the
// window workgroups after them keep their XCD placement.
SWA_HD long long grow_workgroups(long long units) { return units > 0 ? ((units + 1) / 2 + 7) / 8 * 8 : 0; }
SWA_HD long long grow_unit(long long wg, int wave) { return 2 * wg + wave; }

}  // namespace tm
}  // namespace swa
