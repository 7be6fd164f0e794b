// CPU check of the 128 x 128 grouped GEMM's stage-load offsets (mfma_addr.h):
// for one projection shape, every offset a thread forms for operand A, the
// weights and (FP4) both scale operands, at every K-step, must index the
// intended bytes of the intended row or tile, inside the buffer.  Also runs
// the same enumeration through a wrapping formula (the step offset cast to
// 32 bits after the subtraction, then added to a 64-bit address) to show
// that the check sees such a wrap.
//
// usage: mfma_addr_check FP4(0/1) GATEUP(0/1) H I ROWS
// prints "violations N wrapped_violations M"
#include <stdio.h>
#include <stdlib.h>

#include "../../fp4_expert_ffn_amd/csrc/mfma_addr.h"

using namespace moe;

static long long bad = 0;
static void fail(const char* what, long long a, long long b) {
  if (bad++ < 8) fprintf(stderr, "violation: %s (%lld, %lld)\n", what, a, b);
}

// the wrapping form: (uint32_t)(ks * per_step - back) added to the 64-bit base
static unsigned long long wrapped(uint32_t base, int ks, uint32_t per_step, uint32_t back) {
  return (unsigned long long)base + (unsigned long long)(uint32_t)((int)(ks * (int)per_step) - (int)back);
}

int main(int argc, char** argv) {
  if (argc != 6) return 2;
  const int fp4 = atoi(argv[1]), gateup = atoi(argv[2]), H = atoi(argv[3]), I = atoi(argv[4]);
  const long long rows = atoll(argv[5]);  // rows of the A operand buffer (tokens or permuted rows)
  const int K = gateup ? H : I, N = gateup ? 2 * I : H;
  const int kt_vals = fp4 ? 128 : 32;            // values per weight K-tile
  const int step_vals = fp4 ? 256 : 64;          // values per K-step (128 bytes of a row)
  const int nsteps = (K + step_vals - 1) / step_vals;
  const bool half_tail = fp4 && (K % step_vals) != 0;
  const uint32_t arow = fp4 ? K / 2 : K * 2;     // A row bytes
  const unsigned long long abytes = (unsigned long long)rows * arow;
  const int nk_w = K / kt_vals;
  const unsigned long long wbytes = (unsigned long long)(N / 16) * nk_w * 1024;
  const uint32_t srow = K / 32;
  const unsigned long long sabytes = (unsigned long long)rows * srow, sbbytes = (unsigned long long)(N / 16) * nk_w * 64;
  long long wrapped_bad = 0;
  const long long row_probe[3] = {0, rows / 2, rows - 1};
  for (int ks = 0; ks < nsteps; ++ks) {
    const bool tail = half_tail && ks == nsteps - 1;
    for (int tid = 0; tid < 256; ++tid) {
      // ---- A: every probe row, the thread's segment
      for (long long r : row_probe) {
        const uint32_t base = mfma_a_base((uint32_t)r, arow, tid);
        const uint32_t off = mfma_step_off(base, ks, 128u, mfma_a_back(tid, tail));
        const long long in_row = (long long)off - r * arow;
        const long long want = (long long)ks * 128 + (tid & 7) * 16 - ((tail && (tid & 7) >= 4) ? 64 : 0);
        if (in_row != want) fail("A byte within its row", in_row, want);
        if ((unsigned long long)off + 16 > abytes) fail("A past its buffer", off, abytes);
        if (wrapped(base, ks, 128u, mfma_a_back(tid, tail)) + 16 > abytes) ++wrapped_bad;
      }
      // ---- B: every column tile's row groups
      for (int nt = 0; nt < N / 128; ++nt) {
        for (int i = 0; i < 4; ++i) {
          const uint32_t base = mfma_b_base(nt * 8, nk_w, tid, i);
          const uint32_t off = mfma_step_off(base, ks, 2048u, mfma_b_back(tid, tail));
          const long long rg = off / (1024LL * nk_w), kt = (off % (1024LL * nk_w)) / 1024, ln = (off % 1024) / 16;
          const long long want_kt = tail ? 2LL * ks : 2LL * ks + ((tid >> 6) & 1);
          if (rg != nt * 8 + (tid >> 7) + 2 * i) fail("B row group", rg, nt * 8 + (tid >> 7) + 2 * i);
          if (kt != want_kt) fail("B K-tile", kt, want_kt);
          if (ln != (tid & 63)) fail("B lane", ln, tid & 63);
          if ((unsigned long long)off + 16 > wbytes) fail("B past the weights", off, wbytes);
          if (wrapped(base, ks, 2048u, mfma_b_back(tid, tail)) + 16 > wbytes) ++wrapped_bad;
        }
        if (!fp4) continue;
        const uint32_t sb = mfma_step_off(mfma_sb_base(nt * 8, nk_w, tid), ks, 128u, mfma_sb_back(tid, tail));
        const long long srg = sb / (64LL * nk_w), skt = (sb % (64LL * nk_w)) / 64;
        const long long want_skt = tail ? 2LL * ks : 2LL * ks + ((tid >> 4) & 1);
        if (srg != nt * 8 + (tid >> 5)) fail("B scale row group", srg, nt * 8 + (tid >> 5));
        if (skt != want_skt) fail("B scale K-tile", skt, want_skt);
        if ((unsigned long long)sb + 4 > sbbytes) fail("B scales past their section", sb, sbbytes);
      }
      if (!fp4) continue;
      for (long long r : row_probe) {
        const uint32_t sa = mfma_step_off(mfma_sa_base((uint32_t)r, srow, tid), ks, 8u, mfma_sa_back(tid, tail));
        const long long in_row = (long long)sa - r * srow;
        const long long want = (long long)ks * 8 + (tid & 1) * 4 - ((tail && (tid & 1)) ? 4 : 0);
        if (in_row != want) fail("A scale byte within its row", in_row, want);
        if ((unsigned long long)sa + 4 > sabytes) fail("A scales past their buffer", sa, sabytes);
      }
    }
  }
  // ---- weights decoded at the LDS store (bf16 activations): every E2M1
  // (NVFP4 / MXFP4) and FP8 fragment and scale of every step, for every
  // column tile, must be the one the bf16 layout wants and stay in its section
  if (!fp4) {
    const int steps64 = K / 64, nk4 = K / 128, nk8 = K / 64;
    const unsigned long long w4 = (unsigned long long)(N / 16) * nk4 * 1024, w8 = (unsigned long long)(N / 16) * nk8 * 1024;
    for (int nt = 0; nt < N / 128; ++nt)
      for (int ks = 0; ks < steps64; ++ks)
        for (int tid = 0; tid < 256; ++tid) {
          const uint32_t o = mfma_q4_b_off(nt * 8, nk4, tid, ks);
          const long long rg = o / (1024LL * nk4), kt = (o % (1024LL * nk4)) / 1024, ln = (o % 1024) / 16;
          if (rg != nt * 8 + tid / 32 || kt != ks / 2 || ln != 32 * (ks % 2) + tid % 32) fail("E2M1 fragment", o, tid);
          if ((unsigned long long)o + 16 > w4) fail("E2M1 past the weights", o, w4);
          for (uint32_t lsb : {1u, 2u}) {
            const uint32_t so = mfma_q4_s_off(nt * 8, nk4, tid, ks, lsb);
            if (so != (uint32_t)((rg * nk4 + kt) * 64 * lsb + ln * lsb)) fail("E2M1 scale", so, lsb);
            if ((unsigned long long)so + lsb > (unsigned long long)(N / 16) * nk4 * 64 * lsb) fail("scale past", so, lsb);
          }
          for (int i = 0; i < 2; ++i) {
            const uint32_t f = mfma_f8_b_off(nt * 8, nk8, tid, i, ks);
            const int c = tid + 256 * i;
            const long long frg = f / (1024LL * nk8), fkt = (f % (1024LL * nk8)) / 1024, fl = (f % 1024) / 16;
            if (frg != nt * 8 + c / 64 || fkt != ks || fl != c % 64) fail("FP8 fragment", f, c);
            if ((unsigned long long)f + 16 > w8) fail("FP8 past the weights", f, w8);
          }
        }
  }
  printf("violations %lld wrapped_violations %lld\n", bad, wrapped_bad);
  return 0;
}
