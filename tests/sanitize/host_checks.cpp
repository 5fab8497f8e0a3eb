// CPU check of the MoE library's host code (host.cpp): argument validation,
// blob layout, workspace plan and the host packer.  Built with g++ under the
// address and undefined-behaviour sanitizers by tests/test_abi_host.py; any
// sanitizer report or failed check ends the process with a non-zero status.
//
// The packer round trip decodes each blob with this file's own reading of
// the documented layout (include/moe.h, moe_blob_layout_t), not with the
// library's code.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "moe.h"

static int g_fail = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      g_fail = 1;                                                  \
    }                                                              \
  } while (0)

static moe_layer_desc make(int T, int H, int E, int k, int I, int Is, int bits) {
  moe_layer_desc d;
  memset(&d, 0, sizeof d);
  d.n_tokens = T;
  d.hidden = H;
  d.n_experts = E;
  d.top_k = k;
  d.inter = I;
  d.shared_inter = Is;
  d.group = 64;
  d.bits = bits;
  d.act_dtype = MOE_ACT_BF16;
  d.flags = MOE_FLAG_SHARED;
  d.rms_eps = 1e-6f;
  moe_blob_layout_t L;
  if (moe_blob_layout(&d, I, &L) == MOE_OK) d.expert_stride = L.blob_bytes;
  return d;
}

static unsigned lcg(unsigned& s) {
  s = s * 1664525u + 1013904223u;
  return s >> 8;
}

// Decode one (row, col) code and (scale, bias) of a section from the blob.
static void read_elem(const uint8_t* sec, const moe_blob_layout_t& L, int bits, int nmat, int m,
                      int unit_bytes, int tile_bytes, int r, int c, int* code, uint16_t* sc,
                      uint16_t* bi) {
  const int tile = r / L.row_tile, rl = r % L.row_tile;
  const int kb = c / L.kblock_cols, cc = c % L.kblock_cols;
  const uint8_t* unit = sec + (int64_t)tile * tile_bytes + (int64_t)kb * unit_bytes;
  const uint8_t* row = unit + m * 1024 + rl * 64;
  *code = bits == 4 ? (row[cc / 2] >> (4 * (cc & 1))) & 15 : row[cc];
  const int gi = cc / 64;
  const uint8_t* p = unit + nmat * 1024 + m * L.row_tile * L.groups_per_kblock * 4 +
                     (rl * L.groups_per_kblock + gi) * 4;
  memcpy(sc, p, 2);
  memcpy(bi, p + 2, 2);
}

static void packer_round_trip(int bits, int H, int I, bool shared) {
  moe_layer_desc d = make(4, H, 8, 2, I, I, bits);
  moe_blob_layout_t L;
  CHECK(moe_blob_layout(&d, I, &L) == MOE_OK);
  const int qmax = (1 << bits) - 1;
  unsigned s = 12345u + bits + H + I;
  std::vector<uint8_t> qg(I * H), qu(I * H), qd(H * I);
  std::vector<uint16_t> sbg(2 * I * (H / 64)), sbu(2 * I * (H / 64)), sbd(2 * H * (I / 64));
  for (auto& v : qg) v = lcg(s) & qmax;
  for (auto& v : qu) v = lcg(s) & qmax;
  for (auto& v : qd) v = lcg(s) & qmax;
  for (auto& v : sbg) v = (uint16_t)lcg(s);
  for (auto& v : sbu) v = (uint16_t)lcg(s);
  for (auto& v : sbd) v = (uint16_t)lcg(s);
  std::vector<float> wsg(H);
  for (int i = 0; i < H; ++i) wsg[i] = (float)i * 0.5f;
  const int64_t bytes = shared ? L.shared_bytes : L.blob_bytes;
  std::vector<uint8_t> blob(bytes, 0xAB);  // exactly the documented size
  CHECK(moe_pack_expert(&d, I, qg.data(), qu.data(), qd.data(), sbg.data(), sbu.data(),
                        sbd.data(), shared ? wsg.data() : nullptr, blob.data()) == MOE_OK);
  const int G = H / 64, Gd = I / 64;
  for (int r = 0; r < I; ++r)
    for (int c = 0; c < H; ++c)
      for (int m = 0; m < 2; ++m) {
        int code;
        uint16_t sc, bi;
        read_elem(blob.data() + L.gu_offset, L, bits, 2, m, (int)L.gu_unit_bytes,
                  (int)L.gu_tile_bytes, r, c, &code, &sc, &bi);
        const std::vector<uint8_t>& q = m ? qu : qg;
        const std::vector<uint16_t>& sb = m ? sbu : sbg;
        CHECK(code == q[r * H + c]);
        CHECK(sc == sb[r * G + c / 64]);
        CHECK(bi == sb[I * G + r * G + c / 64]);
      }
  for (int r = 0; r < H; ++r)
    for (int c = 0; c < I; ++c) {
      int code;
      uint16_t sc, bi;
      read_elem(blob.data() + L.down_offset, L, bits, 1, 0, (int)L.down_unit_bytes,
                (int)L.down_tile_bytes, r, c, &code, &sc, &bi);
      CHECK(code == qd[r * I + c]);
      CHECK(sc == sbd[r * Gd + c / 64]);
      CHECK(bi == sbd[H * Gd + r * Gd + c / 64]);
    }
  if (shared) CHECK(memcmp(blob.data() + L.shared_gate_offset, wsg.data(), 4 * H) == 0);
  // an out-of-range code is rejected before anything is written
  qd[7] = (uint8_t)(qmax + 1);
  if (bits == 4)
    CHECK(moe_pack_expert(&d, I, qg.data(), qu.data(), qd.data(), sbg.data(), sbu.data(),
                          sbd.data(), nullptr, blob.data()) == MOE_ERR_INVALID_ARG);
}

static void validation() {
  moe_layer_desc ok = make(64, 2048, 512, 10, 512, 512, 4);
  moe_blob_layout_t L;
  CHECK(moe_blob_layout(&ok, ok.inter, &L) == MOE_OK);
  CHECK(moe_workspace_bytes(&ok) > 0);
  CHECK(moe_blob_layout(nullptr, 512, &L) == MOE_ERR_INVALID_ARG);
  CHECK(moe_blob_layout(&ok, 512, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_workspace_bytes(nullptr) == 0);
  struct Mut {
    int field;
    int value;
  };
  // every field through values around its limits; no call may read or write
  // out of bounds whatever it returns
  const int values[] = {-1, 0, 1, 2, 3, 4, 7, 8, 15, 16, 17, 63, 64, 65, 127, 128, 129,
                        255, 256, 384, 512, 1024, 1025, 2048, 4096, 4097, 8192, 8193,
                        1 << 20, 0x7fffffff};
  for (int f = 0; f < 9; ++f)
    for (int v : values) {
      moe_layer_desc d = ok;
      int32_t* fields[] = {&d.n_tokens, &d.hidden, &d.n_experts, &d.top_k, &d.inter,
                           &d.shared_inter, &d.group, &d.bits, &d.act_dtype};
      *fields[f] = v;
      const size_t ws = moe_workspace_bytes(&d);
      (void)moe_blob_layout(&d, d.inter, &L);
      std::vector<uint8_t> fake(64, 0);
      int32_t* pi = nullptr;
      float* pw = nullptr;
      float* pg = nullptr;
      uint32_t* st = nullptr;
      const int r1 = moe_workspace_routing(&d, fake.data(), &pi, &pw, &pg);
      const int r2 = moe_chain_status(&d, fake.data(), &st);
      CHECK((ws == 0) == (r1 != MOE_OK));
      CHECK(r1 == r2);
      if (r1 == MOE_OK) {
        const uint8_t* base = fake.data();
        CHECK((const uint8_t*)pi >= base && (size_t)((const uint8_t*)pi - base) < ws);
        CHECK((const uint8_t*)st >= base && (size_t)((const uint8_t*)st - base) + 4 <= ws);
      }
    }
  // flags and stride
  moe_layer_desc d = ok;
  d.flags = 0x80;
  CHECK(moe_workspace_bytes(&d) == 0);
  uint32_t* st = nullptr;
  CHECK(moe_chain_status(&ok, nullptr, &st) == MOE_ERR_INVALID_ARG);
  CHECK(moe_chain_status(&ok, (void*)0x1000, nullptr) == MOE_ERR_INVALID_ARG);
  // the status word sits after the epoch counter and inside the workspace
  // for every token count
  for (int T : {1, 2, 8, 9, 64, 4096}) {
    moe_layer_desc e = ok;
    e.n_tokens = T;
    const size_t ws = moe_workspace_bytes(&e);
    CHECK(moe_chain_status(&e, (void*)0x100000, &st) == MOE_OK);
    CHECK((uintptr_t)st % 4 == 0);
    CHECK((uintptr_t)st - 0x100000 + 4 <= ws);
  }
}

static void layouts() {
  for (int bits : {4, 8})
    for (int H : {128, 256, 384, 2048, 8192})
      for (int I : {128, 256, 512, 4096}) {
        moe_layer_desc d = make(1, H, 16, 2, I, I, bits);
        moe_blob_layout_t L;
        if (moe_blob_layout(&d, I, &L) != MOE_OK) continue;
        const int64_t codes = 3LL * H * I * bits / 8;
        const int64_t sb = 3LL * H * I / 64 * 4;
        CHECK(L.blob_bytes % 256 == 0 && L.blob_bytes >= codes + sb);
        CHECK(L.blob_bytes - (codes + sb) < 256);
        CHECK(L.down_offset + L.down_tile_bytes * (H / L.row_tile) <= L.blob_bytes);
        CHECK(L.shared_gate_offset + 4LL * H <= L.shared_bytes);
      }
}

// dense blob (MOE_FLAG_DENSE_Q4): pack, then read every code and word back
// at the documented positions
static void dense_round_trip(int H, int E, bool shared) {
  moe_layer_desc d = make(1, H, E, 2, 128, 128, 4);
  d.flags = (shared ? MOE_FLAG_SHARED : 0u) | MOE_FLAG_DENSE_Q4;
  moe_dense_layout_t L;
  CHECK(moe_dense_layout(&d, &L) == MOE_OK);
  const int R = E + (shared ? 1 : 0), G = H / 64;
  CHECK(L.rows == R);
  CHECK(L.words_offset >= (int64_t)R * H / 2 && L.words_offset % 256 == 0);
  CHECK(L.bytes % 256 == 0 && L.bytes >= L.words_offset + 4LL * R * G);
  std::vector<uint8_t> q((size_t)R * H);
  std::vector<uint16_t> sb((size_t)2 * R * G);
  for (size_t i = 0; i < q.size(); ++i) q[i] = (uint8_t)((i * 7 + i / 13) % 16);
  for (size_t i = 0; i < sb.size(); ++i) sb[i] = (uint16_t)(0x3c00 + i * 31);
  std::vector<uint8_t> blob((size_t)L.bytes, 0xAB);
  CHECK(moe_pack_dense(&d, q.data(), sb.data(), blob.data()) == MOE_OK);
  for (int r = 0; r < R; ++r) {
    for (int c = 0; c < H; ++c)
      CHECK(((blob[(size_t)r * H / 2 + c / 2] >> (4 * (c & 1))) & 15) == q[(size_t)r * H + c]);
    for (int g = 0; g < G; ++g) {
      uint32_t w;
      memcpy(&w, blob.data() + L.words_offset + 4 * ((size_t)r * G + g), 4);
      CHECK((w & 0xFFFFu) == sb[(size_t)r * G + g]);
      CHECK((w >> 16) == sb[(size_t)R * G + (size_t)r * G + g]);
    }
  }
  q[5] = 16;
  CHECK(moe_pack_dense(&d, q.data(), sb.data(), blob.data()) == MOE_ERR_INVALID_ARG);
  CHECK(moe_pack_dense(&d, nullptr, sb.data(), blob.data()) == MOE_ERR_INVALID_ARG);
  CHECK(moe_dense_layout(&d, nullptr) == MOE_ERR_INVALID_ARG);
  d.hidden = 96;
  CHECK(moe_dense_layout(&d, &L) == MOE_ERR_UNSUPPORTED);
}

int main() {
  validation();
  layouts();
  dense_round_trip(256, 16, true);
  dense_round_trip(2048, 512, true);
  dense_round_trip(128, 3, false);
  packer_round_trip(4, 256, 128, true);
  packer_round_trip(8, 256, 128, false);
  packer_round_trip(4, 384, 256, false);
  packer_round_trip(8, 128, 64, true);
  if (g_fail) return 1;
  printf("host checks passed\n");
  return 0;
}
