// layout_check.cpp -- host-side check of the LDS tile layouts used by the kernels.
//
// Models, on the CPU, (1) how the direct global->LDS copies fill a tile
// (16-byte slot p of the tile holds logical chunk (p % CH) ^ swz(row) of row
// p / CH), (2) the 16-byte row reads and (3) the gfx950 transposing read
// (within each group of 16 lanes, result lane i, element r is element i % 4
// of the 8 bytes addressed by lane 4r + i/4).  For every MFMA operand the
// kernels build, it checks that each lane receives exactly the logical
// elements its K slots stand for, and that each read is free of LDS bank
// conflicts (64 banks of 4 bytes; a 16-byte read served 16 lanes at a time,
// an 8-byte read 32 lanes at a time).  Exit status 0 = all checks passed.
#include <cstdio>
#include <functional>
#include <set>
#include <vector>

#include "../../exact_tiled_attention_flash_amd/csrc/fa_common.hpp"

using namespace fa;

static int failures = 0;
#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      if (failures < 20) {               \
        std::printf("FAIL: " __VA_ARGS__); \
        std::printf("\n");               \
      }                                  \
      ++failures;                        \
    }                                    \
  } while (0)

// element id = row * D + col, stored per bf16 position of the tile
template <int D>
std::vector<int> tile_image(int rows, const std::function<int(int)>& swz) {
  const int CH = D / 8;
  std::vector<int> img(rows * D);
  for (int p = 0; p < rows * CH; ++p) {
    const int r = p / CH, c = (p % CH) ^ swz(r);
    for (int e = 0; e < 8; ++e) img[p * 8 + e] = r * D + c * 8 + e;
  }
  return img;
}

// max number of distinct 4-byte words mapped to one bank among `lanes`
int bank_conflict_degree(const std::vector<int>& byte_offs, int bytes) {
  std::vector<std::set<int>> bank(64);
  for (int off : byte_offs)
    for (int w = 0; w < bytes / 4; ++w) {
      const int word = off / 4 + w;
      bank[word % 64].insert(word);
    }
  size_t deg = 0;
  for (auto& b : bank) deg = b.size() > deg ? b.size() : deg;
  return (int)deg;
}

template <int D>
void check_row_reads(const char* name, const std::vector<int>& img, int rows,
                     const std::function<int(int, int, int)>& off_fn) {
  for (int r0 = 0; r0 < rows; r0 += 32)
    for (int k = 0; k < D / 16; ++k) {
      std::vector<int> offs(64);
      for (int lane = 0; lane < 64; ++lane) {
        const int g = lane >> 5, r = r0 + (lane & 31);
        const int off = off_fn(r, k, g);
        offs[lane] = off;
        for (int e = 0; e < 8; ++e)
          CHECK(img[off / 2 + e] == r * D + 16 * k + 8 * g + e, "%s D=%d row read r=%d k=%d g=%d e=%d", name, D, r, k, g, e);
      }
      for (int q = 0; q < 4; ++q) {
        std::vector<int> part(offs.begin() + 16 * q, offs.begin() + 16 * q + 16);
        const int deg = bank_conflict_degree(part, 16);
        CHECK(deg == 1, "%s D=%d row read r0=%d k=%d quarter %d: %d-way bank conflict", name, D, r0, k, q, deg);
      }
    }
}

template <int D>
void check_tr_reads(const char* name, const std::vector<int>& img,
                    const std::function<int(int, int, int, int)>& off_fn) {
  for (int t = 0; t < 4; ++t)
    for (int db = 0; db < D / 32; ++db)
      for (int h = 0; h < 2; ++h) {
        std::vector<int> offs(64);
        for (int lane = 0; lane < 64; ++lane) offs[lane] = off_fn(t, db, h, lane);
        for (int lane = 0; lane < 64; ++lane) {
          const int grp = lane / 16, i = lane % 16, g = lane >> 5;
          for (int r = 0; r < 4; ++r) {
            const int sup = 16 * grp + 4 * r + i / 4;
            const int got = img[offs[sup] / 2 + (i % 4)];
            const int want_row = 16 * t + 8 * h + 4 * g + r;
            const int want_col = 32 * db + (lane & 31);
            CHECK(got == want_row * D + want_col, "%s D=%d tr t=%d db=%d h=%d lane=%d slot=%d: got (%d,%d) want (%d,%d)",
                  name, D, t, db, h, lane, 4 * h + r, got / D, got % D, want_row, want_col);
          }
        }
        for (int half = 0; half < 2; ++half) {
          std::vector<int> part(offs.begin() + 32 * half, offs.begin() + 32 * half + 32);
          const int deg = bank_conflict_degree(part, 8);
          CHECK(deg == 1, "%s D=%d tr t=%d db=%d h=%d half %d: %d-way bank conflict", name, D, t, db, h, half, deg);
        }
      }
}

// padded tile filled by the direct copies: 16-byte slot p holds the 16 bytes
// at byte pad_slot_src(p) of the row-major [rows x D] source
template <int D, int STRIDE>
std::vector<int> padded_image(int rows) {
  std::vector<int> img(rows * STRIDE / 2, -1);
  for (int p = 0; p < rows * STRIDE / 16; ++p) {
    const int src = pad_slot_src<D, STRIDE>(p);
    for (int e = 0; e < 8; ++e) img[p * 8 + e] = src / 2 + e;   // element id = row * D + col
  }
  return img;
}

template <int D>
void check_all() {
  // forward (padded): K tile (row reads) and V tile (transposing reads), 64 rows each
  {
    auto kp = padded_image<D, Pad<D>::KSTR>(64);
    check_row_reads<D>("fwd K padded", kp, 64, [](int r, int k, int g) { return row_offset_kpad<D>(r, k, g); });
    auto vp = padded_image<D, Pad<D>::VSTR>(64);
    check_tr_reads<D>("fwd V padded", vp, [](int t, int db, int h, int l) { return tr_offset_vpad<D>(t, db, h, l); });
    CHECK(64 * Pad<D>::KSTR % 1024 == 0 && 64 * Pad<D>::VSTR % 1024 == 0, "padded tiles must be whole 1 KiB copies");
  }
  // forward: K tile (row reads) and V tile (transposing reads), 64 rows each
  auto kimg = tile_image<D>(64, [](int r) { return swz_k<D>(r); });
  check_row_reads<D>("fwd K", kimg, 64, [](int r, int k, int g) { return row_offset_k<D>(r, k, g); });
  auto vimg = tile_image<D>(64, [](int r) { return swz_v<D>(r); });
  check_tr_reads<D>("fwd V", vimg, [](int t, int db, int h, int l) { return tr_offset_v<D>(t, db, h, l); });
  // backward dK/dV: the work-group's 128-row K and V blocks (row reads)
  auto kblk = tile_image<D>(128, [](int r) { return swz_k<D>(r); });
  check_row_reads<D>("bwd K/V block", kblk, 128, [](int r, int k, int g) { return row_offset_k<D>(r, k, g); });
  // backward: the copy mapping of swz_dual tiles matches the modelled layout
  {
    auto dimg2 = tile_image<D>(64, [](int r) { return swz_dual<D>(r); });
    for (int p = 0; p < 64 * D / 8; ++p)
      for (int e = 0; e < 8; ++e)
        CHECK(dimg2[p * 8 + e] == dual_slot_src<D>(p) / 2 + e, "dual_slot_src D=%d slot %d", D, p);
  }
  // backward: padded 128-row K/V block of the dK/dV kernel and padded V tile of the dQ kernel
  {
    auto kb = padded_image<D, Pad<D>::KSTR>(128);
    check_row_reads<D>("bwd K/V block padded", kb, 128, [](int r, int k, int g) { return row_offset_kpad<D>(r, k, g); });
  }
  // backward: tiles read both ways
  auto dimg = tile_image<D>(64, [](int r) { return swz_dual<D>(r); });
  check_row_reads<D>("bwd dual", dimg, 64, [](int r, int k, int g) { return row_offset_dual<D>(r, k, g); });
  check_tr_reads<D>("bwd dual", dimg, [](int t, int db, int h, int l) { return tr_offset_dual<D>(t, db, h, l); });
}

// The fused backward's dS exchange: every wave (kb, qh) of the dK/dV
// work-group writes its 32 keys x 32 queries of dS from the C layout of
// S = Q K^T (lane = key 32kb + l%32, register i = query 8(i/4) + 4(l/32) +
// i%4 of the half), four 8-byte writes per lane; the transposing reads then
// give the A operand of dQ = dS K (lane = query, slots = keys in C-row order).
void check_ds_exchange() {
  std::vector<int> img(128 * 64, -1);   // element id = key * 64 + query
  for (int kb = 0; kb < 4; ++kb)
    for (int qh = 0; qh < 2; ++qh)
      for (int i4 = 0; i4 < 4; ++i4) {
        std::vector<int> offs(64);
        for (int lane = 0; lane < 64; ++lane) {
          const int g = lane >> 5, key = 32 * kb + (lane & 31);
          const int off = ds_offset(key, 8 * qh + 2 * i4 + g);
          offs[lane] = off;
          for (int e = 0; e < 4; ++e) img[off / 2 + e] = key * 64 + 32 * qh + 8 * i4 + 4 * g + e;
        }
        for (int half = 0; half < 2; ++half) {
          std::vector<int> part(offs.begin() + 32 * half, offs.begin() + 32 * half + 32);
          const int deg = bank_conflict_degree(part, 8);
          CHECK(deg == 1, "dS write kb=%d qh=%d i4=%d half %d: %d-way bank conflict", kb, qh, i4, half, deg);
        }
      }
  for (int v : img) CHECK(v >= 0, "dS buffer element never written");
  for (int qh = 0; qh < 2; ++qh)
    for (int t = 0; t < 8; ++t)
      for (int h = 0; h < 2; ++h) {
        std::vector<int> offs(64);
        for (int lane = 0; lane < 64; ++lane) offs[lane] = ds_tr_offset(t, h, qh, lane);
        for (int lane = 0; lane < 64; ++lane) {
          const int grp = lane / 16, i = lane % 16, g = lane >> 5;
          for (int r = 0; r < 4; ++r) {
            const int sup = 16 * grp + 4 * r + i / 4;
            const int got = img[offs[sup] / 2 + (i % 4)];
            const int want = (16 * t + 8 * h + 4 * g + r) * 64 + 32 * qh + (lane & 31);
            CHECK(got == want, "dS tr read qh=%d t=%d h=%d lane=%d r=%d: got (%d,%d) want (%d,%d)", qh, t, h, lane, r,
                  got / 64, got % 64, want / 64, want % 64);
          }
        }
        for (int half = 0; half < 2; ++half) {
          std::vector<int> part(offs.begin() + 32 * half, offs.begin() + 32 * half + 32);
          const int deg = bank_conflict_degree(part, 8);
          CHECK(deg == 1, "dS tr read qh=%d t=%d h=%d half %d: %d-way bank conflict", qh, t, h, half, deg);
        }
      }
}

// The fused backward's K block in the swz_dual layout, 128 rows: row reads
// (S = Q K^T) and the transposing reads of dQ = dS K for all 8 key steps.
template <int D>
void check_dual_block128() {
  auto img = tile_image<D>(128, [](int r) { return swz_dual<D>(r); });
  check_row_reads<D>("bwd K block dual", img, 128, [](int r, int k, int g) { return row_offset_dual<D>(r, k, g); });
  for (int t = 0; t < 8; ++t)
    for (int db = 0; db < D / 32; ++db)
      for (int h = 0; h < 2; ++h)
        for (int lane = 0; lane < 64; ++lane) {
          // key step t is key step 0 shifted by 16t rows: the offset must be additive
          CHECK(tr_offset_dual<D>(t, db, h, lane) == tr_offset_dual<D>(0, db, h, lane) + t * 16 * 2 * D,
                "swz_dual tr offset not additive in t (t=%d db=%d h=%d lane=%d)", t, db, h, lane);
          const int off = tr_offset_dual<D>(t, db, h, lane);
          const int row = 16 * t + 8 * h + 4 * (lane >> 5) + ((lane & 15) >> 2);
          CHECK(img[off / 2] / D == row, "dual block tr t=%d row", t);
        }
}

int main() {
  check_all<128>();
  check_all<64>();
  check_ds_exchange();
  check_dual_block128<128>();
  check_dual_block128<64>();
  if (failures) {
    std::printf("%d layout check(s) failed\n", failures);
    return 1;
  }
  std::printf("layout checks passed\n");
  return 0;
}
