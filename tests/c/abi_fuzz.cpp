// Host fuzz of the C ABI's argument checking, built with AddressSanitizer and
// UBSan (with the kernel launchers stubbed out, tests/c/launch_stubs.cpp) by
// tests/test_host_sanitizers.py.  Random argument vectors -- sizes from
// negative to huge, NULL / aligned / misaligned device pointers (never
// dereferenced on the host), score mods and prefix levels in real host
// memory -- through every entry point.  Each call must return PA_OK, a
// documented negative code or a positive hipError_t, and host memory must
// stay clean.  Exit status 0 = every call behaved.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pagedattn.h"

static int fails = 0;
static void expect_status(int st, const char* what, int iter) {
  const bool ok = st == PA_OK || (st <= -1 && st >= PA_ERR_SCRATCH) || st > 0;
  if (!ok) {
    std::fprintf(stderr, "%s returned %d at iteration %d\n", what, st, iter);
    ++fails;
  }
  if (st != PA_OK && paged_attn_status_string(st) == nullptr) ++fails;
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
  std::mt19937_64 rng(7);
  auto pick = [&](long long n) { return (long long)(rng() % (unsigned long long)n); };
  const int32_t small_vals[] = {-5, -1, 0, 1, 2, 3, 4, 7, 8, 16, 24, 32, 64, 96, 128, 256, 300, 512, 4096, 1 << 20,
                                0x7fffffff};
  auto v32 = [&]() { return small_vals[pick(sizeof(small_vals) / sizeof(small_vals[0]))]; };
  auto ptr = [&]() -> void* {
    switch (pick(24)) {
      case 0: return nullptr;
      case 1: return reinterpret_cast<void*>(0x1008);  // misaligned
      default: return reinterpret_cast<void*>(0x10000);
    }
  };
  auto iptr = [&]() { return static_cast<int32_t*>(ptr()); };
  int counts[3] = {0, 0, 0};  // ok, invalid, hip error
  auto tally = [&](int st) { counts[st == 0 ? 0 : (st < 0 ? 1 : 2)]++; };
  for (int it = 0; it < iters; ++it) {
    pa_score_mods mods;
    mods.window = v32();
    mods.softcap = pick(4) == 0 ? -1.f : (pick(3) == 0 ? 30.f : 0.f);
    mods.alibi_slopes = static_cast<const float*>(pick(2) ? nullptr : ptr());
    mods.prefix_lens = pick(2) ? nullptr : iptr();
    mods.doc_starts = pick(2) ? nullptr : iptr();
    pa_block_mask bm;
    bm.bits = static_cast<const uint32_t*>(pick(6) == 0 ? nullptr : (pick(8) == 0 ? reinterpret_cast<void*>(0x1002)
                                                                                 : ptr()));
    bm.q_block = pick(4) == 0 ? v32() : 1 << pick(8);
    bm.kv_block = pick(4) == 0 ? v32() : 64 << pick(4);
    bm.rows_per_seq = pick(8) == 0 ? v32() : 1 + (int32_t)pick(64);
    bm.words_per_row = pick(8) == 0 ? v32() : 1 + (int32_t)pick(64);
    mods.block_mask = pick(3) == 0 ? &bm : nullptr;
    const pa_score_mods* mp = pick(3) == 0 ? nullptr : &mods;
    // a valid argument set, then a few fields replaced by random values
    int32_t B = 1 + (int32_t)pick(64), Hkv = 1 << pick(4), Hq = Hkv * (1 << pick(4)), D = pick(2) ? 128 : 64;
    int32_t bs = 16 << pick(5), stride = 1 + (int32_t)pick(4096), maxc = (int32_t)pick(40000);
    int32_t split = (int32_t)(pick(3) - 1) * 512, dtype = (int32_t)pick(2);
    int64_t NB = 1 + pick(100000);
    const int nmut = (int)pick(4);
    for (int m = 0; m < nmut; ++m) {
      switch (pick(10)) {
        case 0: B = v32(); break;
        case 1: Hq = v32(); break;
        case 2: Hkv = v32(); break;
        case 3: D = v32(); break;
        case 4: bs = v32(); break;
        case 5: stride = v32(); break;
        case 6: maxc = v32(); break;
        case 7: split = v32(); break;
        case 8: dtype = (int32_t)pick(4) - 1; break;
        default: NB = pick(5) == 0 ? -1 : (int64_t)v32(); break;
      }
    }
    int st;
    switch (pick(10)) {
      case 0:
        st = kv_append(ptr(), ptr(), ptr(), ptr(), iptr(), B, Hkv, D, bs, NB, dtype, nullptr);
        expect_status(st, "kv_append", it);
        break;
      case 1:
        st = kv_copy_blocks(ptr(), ptr(), iptr(), iptr(), B, Hkv, D, bs, NB, dtype, nullptr);
        expect_status(st, "kv_copy_blocks", it);
        break;
      case 2: {
        const size_t ws = paged_attn_decode_workspace_size(B, Hq, Hkv, D, maxc, split);
        (void)paged_attn_decode_split_tokens(B, Hkv, maxc, split);
        st = paged_attn_decode(ptr(), ptr(), ptr(), ptr(), iptr(), stride, iptr(), B, Hq, Hkv, D, bs, NB, maxc, 0.1f,
                               split, mp, ptr(), pick(2) ? ws : (size_t)pick(1 << 20), dtype, nullptr);
        expect_status(st, "paged_attn_decode", it);
        break;
      }
      case 3:
        st = paged_attn_decode_partials(ptr(), ptr(), ptr(), ptr(), iptr(), stride, iptr(), B, Hq, Hkv, D, bs, NB,
                                        maxc, 0.1f, split, mp, ptr(), (size_t)pick(1ll << 40), dtype, nullptr);
        expect_status(st, "paged_attn_decode_partials", it);
        break;
      case 4:
        st = paged_attn_decode_merge(ptr(), iptr(), B, Hq, Hkv, D, maxc, split, mp, ptr(), (size_t)pick(1ll << 40),
                                     dtype, nullptr);
        expect_status(st, "paged_attn_decode_merge", it);
        break;
      case 5:
        st = paged_attn_decode_noalloc(ptr(), ptr(), ptr(), ptr(), iptr(), stride, iptr(), B, Hq, Hkv, D, bs, NB,
                                       maxc, 0.1f, split, mp, dtype, nullptr);
        expect_status(st, "paged_attn_decode_noalloc", it);
        break;
      case 6:
        st = paged_attn_prefill(ptr(), ptr(), iptr(), ptr(), ptr(), iptr(), stride, iptr(), B, maxc, Hq, Hkv, D, bs,
                                NB, 0.1f, (int32_t)pick(3), mp, dtype, nullptr);
        expect_status(st, "paged_attn_prefill", it);
        break;
      case 7: {
        const int32_t tq = pick(4) == 0 ? v32() : (int32_t)std::min<long long>((long long)B * (1 + pick(600)), 0x7fffffff);
        const int32_t ks = pick(3) == 0 ? v32() : (int32_t)(pick(4) - 1) * 64;  // -64 .. 128
        const int32_t maxk = pick(8) == 0 ? v32() : (maxc < (1 << 30) ? maxc + (int32_t)pick(4096) : maxc);
        const size_t ws = paged_attn_prefill_workspace_size(B, tq, maxc, Hq, Hkv, D, maxk, ks, dtype);
        st = paged_attn_prefill_split(ptr(), ptr(), iptr(), tq, ptr(), ptr(), iptr(), stride, iptr(), B, maxc, Hq, Hkv,
                                      D, bs, NB, maxk, ks, 0.1f, (int32_t)pick(3), mp, ptr(),
                                      pick(2) ? ws : (size_t)pick(1 << 20), dtype, nullptr);
        expect_status(st, "paged_attn_prefill_split", it);
        break;
      }
      default: {
        const int L = (int)pick(10);  // levels array of exactly L entries (the caller's contract)
        std::vector<pa_prefix_level> lv((size_t)L);
        for (auto& l : lv) {
          l.group_starts = iptr();
          l.prefix_starts = pick(2) ? nullptr : iptr();
          l.prefix_ends = iptr();
          l.num_groups = v32();
          l.max_group_size = v32();
          l.max_prefix_len = v32();
        }
        const pa_prefix_level* lp = L ? lv.data() : (pick(2) ? nullptr : lv.data());
        const size_t ws = paged_attn_decode_cascade_workspace_size(B, lp, L, Hq, Hkv, D, maxc);
        st = paged_attn_decode_cascade(ptr(), ptr(), ptr(), ptr(), iptr(), stride, iptr(), B, lp, L, Hq, Hkv, D, bs,
                                       NB, maxc, 0.1f, mp, ptr(), pick(2) ? ws : (size_t)pick(1 << 30), dtype, nullptr);
        expect_status(st, "paged_attn_decode_cascade", it);
        break;
      }
    }
    tally(st);
  }
  std::printf("ABI fuzz: %d calls: %d ok (nothing to do), %d rejected on the host, %d reached a launch\n", iters,
              counts[0], counts[1], counts[2]);
  return fails ? 1 : 0;
}
