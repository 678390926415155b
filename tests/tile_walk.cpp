// CPU walk of the prefill kernels' index arithmetic, built from the same
// header the kernels use (swa_tile_math.h).  For each shape read from stdin
// it replays the kernels' loops over workgroups, waves, lanes and tiles and
// prints
//   OOB <what>                 a load outside its buffer resource, or a
//                              resource outside its tensor
//   BAD <row> <key> <what>     a counted key whose LDS row holds other data
//   DUP <row> <key>            a key counted twice for one row
//   R <row> <n> <sum> <sumsq>  the keys a row counts, as sequence positions
//                              (count, sum, sum of squares)
//   END
// The Python test compares the R lines with the fp64 oracle's masks.
//
// Input lines (one shape each):
//   tiled MODE Tseq W dil pstart D G g_1 .. g_G
//   tiledf32 MODE Tseq W dil pstart D G g_1 .. g_G   (the fp32 matrix-core
//                              kernel: MODE 0/1/2/5/6, any dilation)
//   short MODE T W D
//   grows MODE T D G g_1 .. g_G
// MODE of "tiled" is the tiled kernel's: 0 causal, 1 symmetric, 2 causal
// chunk (Tseq = chunk length, pstart = its first position), 3/4 dilated,
// 5/6 window plus globals, 7/8 dilated window plus globals.

#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <string>
#include <vector>

#include "swa_tile_math.h"

namespace tw = swa::tm;

namespace {

using Keys = std::map<long long, std::set<long long>>;  // row position -> key positions

void swz_check(int D) {
  if (D != 32 && D != 64 && D != 128) {
    std::printf("OOB unsupported head size %d\n", D);
  }
}

void emit(const Keys& keys) {
  for (const auto& kv : keys) {
    long long n = 0, s = 0, s2 = 0;
    for (long long k : kv.second) {
      ++n;
      s += k;
      s2 += k * k;
    }
    std::printf("R %lld %lld %lld %lld\n", kv.first, n, s, s2);
  }
}

void count(Keys& keys, long long row, long long key) {
  if (!keys[row].insert(key).second) std::printf("DUP %lld %lld\n", row, key);
}

// The tiled kernel (prefill_bf16_kernel) for one query head; with f32, the
// fp32 matrix-core kernel (prefill_f32_mfma_kernel): 4-byte elements, every
// window tile crossing an edge masked by the direct test (its global tiles
// count the keys global_counts admits, as the class test of the bf16 kernel).
void walk_tiled(int MODE, int Tseq, int W, int dil, int pstart, int D, const std::vector<int>& gpos,
                bool f32 = false) {
  const bool kCausal = MODE != 1 && MODE != 4 && MODE != 6 && MODE != 8;
  const bool kChunk = MODE == 2;
  const bool kDil = MODE == 3 || MODE == 4 || MODE == 7 || MODE == 8;
  const bool kGlobal = MODE >= 5;
  if (!kDil) dil = 1;
  if (!kChunk) pstart = 0;
  const int ngl = kGlobal ? (int)gpos.size() : 0;
  const int ROWB = D * (f32 ? 4 : 2);
  const int TILEB = tw::kBN * ROWB;
  const int kThreads = 256;
  const int NLD = TILEB / (kThreads * 16);
  const int hw = W >> 1;
  // buffer extents in bytes: one head of K (or V) of Tseq rows; the ring of
  // W slots in the chunk mode
  const long long head_bytes = (long long)Tseq * ROWB;
  const long long ring_bytes = (long long)W * ROWB;
  Keys keys;
  const int n_cls = kDil ? dil : 1;
  for (int cls = 0; cls < n_cls; ++cls) {
    const int T = kDil ? tw::class_rows(Tseq, cls, dil) : Tseq;
    const int RS = kDil ? dil * D : D;  // elements between consecutive rows
    const int RSB = RS * 2;
    const int n_qtiles = ((kDil ? (Tseq + dil - 1) / dil : Tseq) + tw::kBM - 1) / tw::kBM;
    for (int qt = 0; qt < n_qtiles; ++qt) {
      const int q0 = qt * tw::kBM;
      if (kDil && q0 >= T) continue;  // past the end of this class
      int lo, hi;
      if (kCausal) {
        lo = SWA_TM_CAUSAL_BLOCK_LO(q0, W, pstart);
        hi = SWA_TM_CAUSAL_BLOCK_HI(q0, T);
      } else {
        lo = SWA_TM_SYM_BLOCK_LO(q0, hw);
        hi = SWA_TM_SYM_BLOCK_HI(q0, T, hw);
      }
      const int kt0 = kChunk ? tw::floor_tile(lo) : lo / tw::kBN;
      const int kt1 = hi / tw::kBN;
      const int kt_end = kGlobal ? tw::global_tiles_end(kt1, ngl) : kt1;
      // ---- every tile of [kt0, kt_end] is loaded once: check its loads
      for (int kt = kt0; kt <= kt_end; ++kt) {
        const int kbase = kt * tw::kBN;
        for (int tid = 0; tid < kThreads; ++tid) {
          for (int j = 0; j < NLD; ++j) {
            const int o = tw::load_lds_offset(j, tid, kThreads);
            if (o + 16 > TILEB) std::printf("OOB lds offset %d tile %d\n", o, TILEB);
            const int row = tw::load_row(o, ROWB);
            const int chunk = tw::load_chunk(o, ROWB);
            if (chunk < 0 || chunk * 16 + 16 > ROWB) std::printf("OOB chunk %d\n", chunk);
            if (kGlobal && kt > kt1) {
              const int t0 = (kt - kt1 - 1) * tw::kBN;
              const int gi = tw::global_index(t0, row, ngl);
              if (gi < 0 || gi >= ngl) std::printf("OOB global index %d of %d\n", gi, ngl);
              const int gp = tw::global_src_row(gpos[gi], Tseq);
              const long long off = (long long)gp * ROWB + chunk * 16;
              if (off < 0 || off + 16 > head_bytes) std::printf("OOB global load %lld of %lld\n", off, head_bytes);
              continue;
            }
            if (kChunk && kbase < 0) {
              const unsigned slot = tw::ring_slot(pstart, kbase, row, W);
              const long long off = (long long)slot * ROWB + chunk * 16;
              if (off + 16 > ring_bytes) std::printf("OOB ring load %lld of %lld\n", off, ring_bytes);
              continue;
            }
            const int last = tw::tile_last(T, kt);
            const int bytes = tw::tile_bytes(last, RSB, ROWB);
            const long long off = tw::tile_row_offset(row, last, RSB) + chunk * 16;
            if (last < 0) std::printf("OOB tile %d past the rows (last %d)\n", kt, last);
            if (off < 0 || off + 16 > bytes) std::printf("OOB tile load %lld of %d\n", off, bytes);
            // the resource [base, base + bytes) inside the head (or class) rows
            const long long base = (long long)cls * ROWB + (long long)kbase * RSB;
            if (base < 0 || base + bytes > head_bytes) {
              std::printf("OOB tile resource %lld + %d of %lld\n", base, bytes, head_bytes);
            }
          }
        }
      }
      // ---- the keys each row counts
      for (int wave = 0; wave < 4; ++wave) {
        const int qw0 = q0 + wave * 32;
        const bool wave_active = qw0 < T;
        const int qlast = SWA_TM_WAVE_LAST(qw0, T);
        const int wlo = SWA_TM_WAVE_LO(kCausal, qw0, W, hw, pstart);
        const int whi = SWA_TM_WAVE_HI(kCausal, qlast, T, hw);
        for (int lane = 0; lane < 64; ++lane) {
          const int half = lane >> 5;
          const int qi = qw0 + (lane & 31);
          if (qi >= T) continue;  // never stored
          const long long rpos = kChunk ? (long long)pstart + qi : (long long)cls + (long long)dil * qi;
          auto key_pos = [&](int key) {
            return kChunk ? (long long)pstart + key : (long long)cls + (long long)dil * key;
          };
          for (int kt = kt0; kt <= kt1; ++kt) {
            const int k0 = kt * tw::kBN;
            if (!tw::tile_visited(wave_active, wlo, whi, k0)) continue;
            const bool full = tw::tile_full(kCausal, kChunk, k0, qw0, qlast, T, W, pstart);
            // symmetric edge tiles: the class of each 32-key block, as the
            // kernel branches on it (a block no row sees is skipped, a block
            // every row sees is taken unmasked)
            int cls_blk[2] = {tw::kSymSome, tw::kSymSome};
            if (!f32 && !full && !kCausal && tw::sym_blocks_classified(D)) {
              cls_blk[0] = tw::sym_block_class(k0, qw0, qlast, T, W);
              cls_blk[1] = tw::sym_block_class(k0 + 32, qw0, qlast, T, W);
              // a lone block is always masked
              if (cls_blk[1] == tw::kSymNone && cls_blk[0] != tw::kSymNone) cls_blk[0] = tw::kSymSome;
              if (cls_blk[0] == tw::kSymNone && cls_blk[1] != tw::kSymNone) cls_blk[1] = tw::kSymSome;
            }
            for (int mb = 0; mb < 2; ++mb) {
              if (!full && !kCausal && cls_blk[mb] == tw::kSymNone) continue;  // skipped
              for (int r = 0; r < 16; ++r) {
                const int kcn = mb * 32 + 8 * (r >> 2) + (r & 3);  // without the half
                const int kc = kcn + 4 * half;
                const int key = k0 + kc;
                bool ok;
                if (full) {
                  ok = true;
                } else if (f32) {
                  ok = tw::edge_visible(kCausal, qi, key, T, W, pstart);
                } else if (!kCausal && cls_blk[mb] == tw::kSymAll) {
                  ok = true;
                } else if (!kCausal) {
                  ok = tw::sym_visible(tw::sym_range(qi, k0, half, T, W), kcn);
                } else if (!kChunk) {
                  ok = tw::causal_edge_visible(qi - k0, kc, tw::causal_edge_span(qi, W));
                } else {
                  ok = tw::edge_visible(kCausal, qi, key, T, W, pstart);
                }
                if (!ok) continue;
                // the LDS row holds this key's data only if it was not clamped
                if (key > T - 1) std::printf("BAD %lld %d past the end\n", rpos, key);
                if (kChunk && key < 0 && (pstart + key < 0 || key < -W)) {
                  std::printf("BAD %lld %d not in the ring\n", rpos, key);
                }
                count(keys, rpos, key_pos(key));
              }
            }
          }
          if (kGlobal) {
            for (int kt = kt1 + 1; kt <= kt_end; ++kt) {
              const int t0 = (kt - kt1 - 1) * tw::kBN;
              const int nblk = ngl - t0 > 32 ? 2 : 1;
              // the wave's class against this tile (lane j looks at key t0 + j)
              unsigned long long vmask = 0;
              int gmin = 0x7fffffff, gmax = -0x7fffffff - 1;
              for (int j = 0; j < 64; ++j) {
                const int gl = gpos[tw::global_index(t0, j, ngl)];
                if (tw::global_valid(t0 + j, gl, ngl, Tseq)) {
                  vmask |= 1ull << j;
                  gmin = tw::imin(gmin, gl);
                  gmax = tw::imax(gmax, gl);
                }
              }
              const int rlo = kDil ? cls + dil * qw0 : qw0;
              const int rhi = kDil ? cls + dil * qlast : qlast;
              const int wcls = tw::global_wave_class(kCausal, rlo, rhi, gmin, gmax, W, dil);
              unsigned okbits = 0;
              if (wcls == tw::kGlobalAll) {
                okbits = tw::global_lane_bits(vmask, half);
              } else if (wcls == tw::kGlobalSome) {
                for (int g = 0; g < 8; ++g) {
                  for (int e = 0; e < 4; ++e) {
                    const int kl = 8 * g + 4 * half + e;
                    const int gp = gpos[tw::global_index(t0, kl, ngl)];
                    if (tw::global_counts(kCausal, kDil, (int)rpos, gp, t0 + kl, ngl, Tseq, W, dil)) {
                      okbits |= 1u << (4 * g + e);
                    }
                  }
                }
              }
              for (int g = 0; g < 4 * nblk; ++g) {
                for (int e = 0; e < 4; ++e) {
                  if (!((okbits >> (4 * g + e)) & 1u)) continue;
                  const int kl = 8 * g + 4 * half + e;
                  const int gp = gpos[tw::global_index(t0, kl, ngl)];
                  // the kernel's per-key test is the reference for the class
                  if (!tw::global_counts(kCausal, kDil, (int)rpos, gp, t0 + kl, ngl, Tseq, W, dil)) {
                    std::printf("BAD %lld global key %d counted by the wave class\n", rpos, gp);
                  }
                  count(keys, rpos, gp);
                }
              }
            }
          }
        }
      }
    }
  }
  emit(keys);
}

// The short-window kernel (prefill_short_kernel) for one query head.
void walk_short(int MODE, int T, int W, int D) {
  const bool causal = MODE == 0;
  const int ROWB = D * 2;
  const int off = causal ? 32 : 16;
  const long long head_bytes = (long long)T * ROWB;
  Keys keys;
  for (int wt = 0; wt * 32 < T; ++wt) {
    const int qw0 = wt * 32;
    const tw::ShortBlock sb = tw::short_block(qw0, off, T);
    const int bytes = (sb.bhi - sb.blo + 1) * ROWB;
    if (sb.blo < 0 || sb.bhi >= T || sb.bhi < sb.blo) std::printf("OOB short block %d..%d\n", sb.blo, sb.bhi);
    if ((long long)sb.blo * ROWB + bytes > head_bytes) std::printf("OOB short resource\n");
    for (int row = 0; row < 64; ++row) {
      for (int chunk = 0; chunk < ROWB / 16; ++chunk) {
        const int src = tw::short_src_row(sb, row);
        const int o = (src - sb.blo) * ROWB + chunk * 16;
        if (o < 0 || o + 16 > bytes) std::printf("OOB short load %d of %d\n", o, bytes);
      }
    }
    for (int lane = 0; lane < 64; ++lane) {
      const int half = lane >> 5;
      const int qi = qw0 + (lane & 31);
      if (qi >= T) continue;
      const tw::ShortMask m = tw::short_mask(causal, qi, sb.kb0, T, W);
      for (int mb = 0; mb < 2; ++mb) {
        for (int r = 0; r < 16; ++r) {
          const int kc = mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (!tw::short_visible(m, kc)) continue;
          const int key = sb.kb0 + kc;
          if (key < 0 || key > T - 1) std::printf("BAD %d %d clamped row\n", qi, key);
          count(keys, qi, key);
        }
      }
    }
  }
  emit(keys);
}

// The global-row units (global_rows_unit) for one query head: every
// global row, over all splits.
void walk_grows(int MODE, int T, int D, const std::vector<int>& gpos) {
  const bool causal = MODE == 0;
  const int ROWB = D * 2;
  const int kRowKeys = 128;
  const int S = (T + kRowKeys - 1) / kRowKeys;
  const long long head_bytes = (long long)T * ROWB;
  // the units of one KV head with G global rows (one chunk of 32 pairs per
  // head here), two per leading workgroup: each exactly once
  {
    const long long units = (long long)S * (((long long)gpos.size() + 31) / 32);
    std::vector<int> seen(units, 0);
    const long long wgs = tw::grow_workgroups(units);
    if (units > 0 && (wgs % 8 != 0 || 2 * wgs < units)) std::printf("BAD row workgroups %lld for %lld units\n", wgs, units);
    for (long long wg = 0; wg < wgs; ++wg) {
      for (int wave = 0; wave < 2; ++wave) {
        const long long u = tw::grow_unit(wg, wave);
        if (u < units) ++seen[u];
      }
    }
    for (long long u = 0; u < units; ++u) {
      if (seen[u] != 1) std::printf("BAD row unit %lld run %d times\n", u, seen[u]);
    }
  }
  Keys keys;
  for (int split = 0; split < S; ++split) {
    const int s0 = tw::grow_split_begin(split, kRowKeys);
    const int s1 = tw::grow_split_end(split, kRowKeys, T);
    // one wave per 32 rows: here each row on its own (the wave's key limit is
    // the largest of its rows' and only adds masked keys)
    for (int gp0 : gpos) {
      const int gp = (gp0 < 0 || gp0 >= T) ? -1 : gp0;
      const int lim = tw::grow_row_limit(causal, gp, T, s1);
      for (int k0 = s0; k0 <= lim; k0 += tw::kBN) {
        for (int row = 0; row < tw::kBN; ++row) {
          const long long o = (long long)tw::grow_src_row(k0, row, T) * ROWB;
          if (o < 0 || o + ROWB > head_bytes) std::printf("OOB grows load %lld of %lld\n", o, head_bytes);
          const int key = k0 + row;
          if (key > lim) continue;
          if (key > T - 1) std::printf("BAD %d %d clamped row\n", gp, key);
          count(keys, gp, key);
        }
      }
    }
  }
  emit(keys);
}

}  // namespace

int main() {
  char kind[16];
  while (std::scanf("%15s", kind) == 1) {
    const std::string k(kind);
    if (k == "tiled") {
      int mode, Tseq, W, dil, pstart, D, G;
      if (std::scanf("%d %d %d %d %d %d %d", &mode, &Tseq, &W, &dil, &pstart, &D, &G) != 7) return 2;
      std::vector<int> g(G);
      for (int i = 0; i < G; ++i)
        if (std::scanf("%d", &g[i]) != 1) return 2;
      swz_check(D);
      walk_tiled(mode, Tseq, W, dil, pstart, D, g);
    } else if (k == "tiledf32") {
      int mode, Tseq, W, dil, pstart, D, G;
      if (std::scanf("%d %d %d %d %d %d %d", &mode, &Tseq, &W, &dil, &pstart, &D, &G) != 7) return 2;
      if (mode != 0 && mode != 1 && mode != 2 && mode != 5 && mode != 6) return 2;
      std::vector<int> g(G);
      for (int i = 0; i < G; ++i)
        if (std::scanf("%d", &g[i]) != 1) return 2;
      swz_check(D);
      // the kernel runs dilations > 1 as the residue-class walks of the bf16
      // kernel's dilated modes (3/4, and 7/8 with global keys)
      int wmode = mode;
      if (dil > 1 && mode < 2) wmode = mode + 3;
      if (dil > 1 && mode >= 5) wmode = mode + 2;
      walk_tiled(wmode, Tseq, W, dil, pstart, D, g, true);
    } else if (k == "short") {
      int mode, T, W, D;
      if (std::scanf("%d %d %d %d", &mode, &T, &W, &D) != 4) return 2;
      walk_short(mode, T, W, D);
    } else if (k == "grows") {
      int mode, T, D, G;
      if (std::scanf("%d %d %d %d", &mode, &T, &D, &G) != 4) return 2;
      std::vector<int> g(G);
      for (int i = 0; i < G; ++i)
        if (std::scanf("%d", &g[i]) != 1) return 2;
      walk_grows(mode, T, D, g);
    } else {
      return 2;
    }
    std::printf("END\n");
    std::fflush(stdout);
  }
  return 0;
}
