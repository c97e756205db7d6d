// Host-side fuzz of the library's planning and validation (built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code by
// tests/test_host_sanitizers.py; no GPU needed, no kernel is launched).
// Random shapes and tile maps, valid and invalid, go through
// h3_workspace_bytes, h3_workspace_layout, h3_denoise_workspace_bytes and
// the argument checks of the entry points (NULL device pointers, so every
// call must return an error before any launch).  Invariants of a valid plan
// are checked too: offsets 256-byte aligned and inside the total, the total
// equal to h3_workspace_bytes.  Exit status: 0, or 1 with a message.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "h3.h"

namespace {

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {  // SplitMix64 (Steele, Lea, Flood 2014)
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int uni(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }
bool coin(int pct) { return uni(0, 99) < pct; }

int failures = 0;
#define EXPECT(cond, ...)                      \
  do {                                         \
    if (!(cond)) {                             \
      fprintf(stderr, "FAIL: " __VA_ARGS__);   \
      fprintf(stderr, "\n");                   \
      ++failures;                              \
    }                                          \
  } while (0)

// a tile map over the three segments: runs of `tile` rows per segment with a
// ragged last tile, optionally broken (non-monotone, straddling, oversized)
void make_tiles(const h3_shape& s, int tile, int breakage, std::vector<int32_t>& ts, int& npt) {
  ts.clear();
  ts.push_back(0);
  int row = 0;
  const int segs[3] = {s.n_text, s.n_audio, s.n_video};
  npt = 0;
  for (int g = 0; g < 3; ++g) {
    const int end = row + segs[g];
    while (row < end) {
      row = row + tile < end ? row + tile : end;
      ts.push_back(row);
    }
    if (g == 1) npt = (int)ts.size() - 1;
  }
  if (breakage == 1 && ts.size() > 3) std::swap(ts[1], ts[2]);              // not monotone
  if (breakage == 2 && ts.size() > 2) ts[ts.size() / 2] += 1;               // an edge off by one
  if (breakage == 3) ts.back() += 7;                                        // past the last row
  if (breakage == 4 && npt > 0) npt -= 1;                                   // prefix edge mid-segment
  if (breakage == 5 && ts.size() > 2) ts[1] = ts[0];                        // an empty tile
}

}  // namespace

int main(int argc, char** argv) {
  const int n_cases = argc > 1 ? atoi(argv[1]) : 3000;
  EXPECT(h3_abi_version() == H3_ABI_VERSION, "abi version %d", h3_abi_version());
  int valid = 0, invalid = 0;
  for (int c = 0; c < n_cases; ++c) {
    h3_shape s{};
    s.n_text = uni(0, 3) == 0 ? 0 : uni(1, 700);
    s.n_audio = uni(0, 3) == 0 ? 0 : uni(1, 700);
    s.n_video = uni(0, 5) == 0 ? 0 : uni(1, 6000);
    s.hidden = 256 * uni(1, 8) + (coin(5) ? uni(-3, 3) : 0);
    s.head_dim = coin(90) ? (coin(50) ? 64 : 128) : uni(1, 200);
    s.n_heads = uni(1, 12);
    s.ffn = 256 * uni(1, 12) + (coin(5) ? 8 : 0);
    s.top_k = coin(10) ? uni(-2, 0) : uni(1, 600);
    s.pooled = uni(0, 1);
    s.norm_eps = 1e-6f;
    s.mlp = coin(95) ? uni(0, 1) : uni(2, 5);
    s.gate = coin(95) ? uni(0, 1) : 7;
    const int tile = coin(95) ? (coin(50) ? 64 : uni(1, 200)) : uni(-5, 0);
    std::vector<int32_t> ts;
    int npt = 0;
    if (tile > 0) {
      make_tiles(s, tile, coin(70) ? 0 : uni(1, 5), ts, npt);
    } else {
      ts = {0, s.n_text + s.n_audio + s.n_video};
    }
    s.n_tiles = coin(97) ? (int)ts.size() - 1 : uni(-1, 5000);
    s.n_prefix_tiles = coin(97) ? npt : uni(-2, 3000);
    const int32_t* tsp = coin(2) ? nullptr : ts.data();
    if (s.n_tiles > (int)ts.size() - 1) tsp = nullptr;  // (the ABI reads n_tiles + 1 entries)

    for (int which = -1; which <= 4; ++which) {
      const size_t bytes = h3_workspace_bytes(&s, tsp, which);
      h3_ws_layout L;
      memset(&L, 0x5a, sizeof(L));
      const int rc = h3_workspace_layout(&s, tsp, which, &L);
      EXPECT((bytes != 0) == (rc == H3_OK), "case %d which %d: bytes %zu but rc %d", c, which,
             bytes, rc);
      if (rc != H3_OK) {
        ++invalid;
        continue;
      }
      ++valid;
      EXPECT(L.total == bytes, "case %d which %d: layout total %zu != %zu", c, which, L.total,
             bytes);
      const size_t offs[] = {L.tables, L.norm, L.big, L.q, L.k, L.vt, L.qbar, L.kbar, L.vbar,
                             L.scores, L.sel, L.pooled, L.attn, L.x1};
      for (size_t o : offs) {
        EXPECT(o % 256 == 0, "case %d which %d: offset %zu not 256-aligned", c, which, o);
        EXPECT(o < L.total, "case %d which %d: offset %zu past total %zu", c, which, o, L.total);
      }
    }
    if (tsp) {  // the denoise plan, and entry points refusing NULL device pointers
      (void)h3_denoise_workspace_bytes(&s, tsp, uni(-1, 60));
      int rc = h3_block_forward(&s, tsp, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                nullptr);
      EXPECT(rc != H3_OK, "case %d: block_forward accepted NULL pointers", c);
      rc = h3_routed_attn(&s, tsp, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, 0, nullptr);
      EXPECT(rc != H3_OK, "case %d: routed_attn accepted NULL pointers", c);
    }
  }
  // row counts whose int32 sum wraps: refused, with no signed overflow on the way
  {
    h3_shape s{};
    s.n_text = 64;
    s.n_audio = 0x7fffffff;
    s.n_video = 0x7fffffff;
    s.hidden = 256;
    s.n_heads = 4;
    s.head_dim = 64;
    s.ffn = 256;
    s.n_tiles = 1;
    s.top_k = 1;
    const int32_t ts[2] = {0, 64};
    EXPECT(h3_workspace_bytes(&s, ts, H3_WS_BLOCK) == 0, "huge row counts accepted");
    EXPECT(h3_rows_in(&s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) != H3_OK,
           "rows_in accepted huge row counts");
  }
  printf("plan fuzz: %d cases, %d valid plans, %d refused, %d failures\n", n_cases, valid,
         invalid, failures);
  return failures == 0 ? 0 : 1;
}
