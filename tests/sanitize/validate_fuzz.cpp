// Host-side descriptor validation under AddressSanitizer and
// UndefinedBehaviorSanitizer: every field of a valid descriptor is set in turn
// to boundary and extreme values (and pairs of fields at once), and the
// validators run on each. Any signed overflow, out-of-range shift or invalid
// memory access aborts the program (-fno-sanitize-recover=all).
#include <math.h>
#include <stdio.h>
#include <stdint.h>

#include <limits>
#include <vector>

#include "validate.h"

using namespace mlra;

static const int32_t kInts[] = {0, 1, -1, 2, 7, 8, 15, 16, 17, 31, 32, 64, 128, 255, 256, 257, 511, 512, 513,
                                1024, 4096, 4097, 65535, 65536, 1 << 20, 1 << 30, INT32_MAX - 1, INT32_MAX,
                                INT32_MIN, INT32_MIN + 1};
static const float kFloats[] = {0.f, -1.f, 1.f, 1e-30f, 1e30f, INFINITY, -INFINITY, NAN};

static int run(const mlra_desc& d, long* ok) {
  ShapeInfo s;
  const int st = check_desc(&d, &s);
  if (st == MLRA_OK) {
    ++*ok;
    // what the library computes from a validated descriptor
    volatile int rb = fp8_mode(&d) ? fp8_row_bytes(&d) : 0;
    volatile int64_t row = static_cast<int64_t>(d.d_c) + d.d_r;
    (void)rb;
    (void)row;
    if (s.w <= 0 || s.hpb <= 0 || s.head_tiles <= 0 || s.hk <= 0 || (1 << s.log2_page) != d.page_size) return 1;
  }
  (void)check_append(&d);
  (void)fp8_mode(&d);
  return 0;
}

int main() {
  std::vector<mlra_desc> bases;
  mlra_desc b{};
  b.batch = 32; b.n_heads = 64; b.d_h = 128; b.d_c = 512; b.n_blocks = 4; b.blocks_per_head = 1; b.d_r = 64;
  b.page_size = 64; b.max_pages_per_seq = 128; b.num_pages = 4097; b.d_model = 4096; b.dtype = MLRA_BF16;
  b.d_cq = 1536;
  for (int dt = 0; dt < 4; ++dt) {
    mlra_desc c = b;
    c.dtype = dt;
    bases.push_back(c);
  }
  long checked = 0, ok = 0;
  int bad = 0;
  for (const mlra_desc& base : bases) {
    int32_t mlra_desc::*ints[] = {&mlra_desc::batch, &mlra_desc::n_heads, &mlra_desc::d_h, &mlra_desc::d_c,
                                  &mlra_desc::n_blocks, &mlra_desc::blocks_per_head, &mlra_desc::d_r,
                                  &mlra_desc::page_size, &mlra_desc::max_pages_per_seq, &mlra_desc::num_pages,
                                  &mlra_desc::d_model, &mlra_desc::dtype, &mlra_desc::d_cq};
    float mlra_desc::*floats[] = {&mlra_desc::softmax_scale, &mlra_desc::out_scale, &mlra_desc::cache_scale,
                                  &mlra_desc::rope_base};
    const int ni = sizeof(ints) / sizeof(ints[0]);
    for (int f = 0; f < ni; ++f)
      for (int32_t v : kInts) {
        mlra_desc d = base;
        d.*ints[f] = v;
        bad += run(d, &ok);
        ++checked;
        // and every second field at every value as well
        for (int g = f + 1; g < ni; ++g)
          for (int32_t u : kInts) {
            mlra_desc e = d;
            e.*ints[g] = u;
            bad += run(e, &ok);
            ++checked;
          }
      }
    for (auto fl : floats)
      for (float v : kFloats) {
        mlra_desc d = base;
        d.*fl = v;
        bad += run(d, &ok);
        ++checked;
      }
  }
  bad += check_desc(nullptr, nullptr) == MLRA_ERR_INVALID_ARG ? 0 : 1;
  bad += check_append(nullptr) == MLRA_ERR_INVALID_ARG ? 0 : 1;
  printf("descriptors checked %ld, valid %ld, inconsistent %d\n", checked, ok, bad);
  return bad == 0 ? 0 : 1;
}
