// Sanitizer run of the library's host-only entry points (built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py).  Every output buffer is
// allocated to its exact size, so a write past it is reported.  Exit status 0 when every call
// returned the expected status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "audio_encoder.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static encoder_cfg full_cfg() {
  encoder_cfg c;
  std::memset(&c, 0, sizeof c);
  c.sample_rate = 16000; c.n_fft = 400; c.hop = 160; c.n_mels = 128; c.conv_channels = 480;
  c.d_model = 1280; c.n_layers = 32; c.n_heads = 20; c.head_dim = 64; c.d_ffn = 5120;
  c.window_tokens = 100; c.d_out = 2048; c.d_adapter = 8192; c.piece_tokens = 800;
  c.dtype = ENC_BF16; c.ln_eps = 1e-5f; c.max_tokens_per_pass = 8192; c.weight_bits = 16;
  return c;
}
static encoder_cfg tiny_cfg() {
  encoder_cfg c = full_cfg();
  c.conv_channels = 32; c.d_model = 256; c.n_layers = 2; c.n_heads = 4; c.d_ffn = 1024;
  c.window_tokens = 25; c.d_out = 512; c.d_adapter = 1024; c.dtype = ENC_F32;
  return c;
}

static void plans(const encoder_cfg& c, const std::vector<int64_t>& lens, int32_t ppp) {
  const int32_t n = (int32_t)lens.size();
  int32_t nw = 0, np = 0;
  const encoder_status st = encoder_plan_windows_ragged(&c, lens.data(), n, nullptr, 0, &nw);
  if (st != ENC_OK) {
    EXPECT(encoder_plan_passes(&c, lens.data(), n, ppp, nullptr, 0, &np) == st);
    return;
  }
  int32_t* tab = new int32_t[7 * (size_t)nw];
  EXPECT(encoder_plan_windows_ragged(&c, lens.data(), n, tab, nw, &nw) == ENC_OK);
  int64_t tok = 0;
  for (int32_t i = 0; i < nw; ++i) tok += tab[7 * i + 5];
  if (ppp == 0 || n == 1) {
    EXPECT(encoder_plan_passes(&c, lens.data(), n, ppp, nullptr, 0, &np) == ENC_OK);
    int64_t* ps = new int64_t[6 * (size_t)np];
    EXPECT(encoder_plan_passes(&c, lens.data(), n, ppp, ps, np, &np) == ENC_OK);
    int64_t w = 0, t = 0;
    for (int32_t i = 0; i < np; ++i) {
      EXPECT(ps[6 * i] == w && ps[6 * i + 2] == t);
      w += ps[6 * i + 1];
      t += ps[6 * i + 3];
    }
    EXPECT(w == nw && t == tok);
    // a short table: only max_passes entries are written
    if (np > 1) {
      int64_t* one = new int64_t[6];
      EXPECT(encoder_plan_passes(&c, lens.data(), n, ppp, one, 1, &np) == ENC_OK);
      delete[] one;
    }
    delete[] ps;
  }
  if (n == 1) {
    int32_t nb = 0;
    EXPECT(encoder_plan_windows(&c, lens[0], 1, nullptr, 0, &nb) == ENC_OK && nb == nw);
    int32_t* t1 = new int32_t[7 * (size_t)nb];
    EXPECT(encoder_plan_windows(&c, lens[0], 1, t1, nb, &nb) == ENC_OK);
    EXPECT(std::memcmp(t1, tab, 7 * sizeof(int32_t) * (size_t)nb) == 0);
    delete[] t1;
  }
  delete[] tab;
}

int main() {
  const encoder_cfg full = full_cfg(), tiny = tiny_cfg();
  EXPECT(encoder_validate_cfg(&full) == ENC_OK);
  EXPECT(encoder_validate_cfg(&tiny) == ENC_OK);
  EXPECT(encoder_validate_cfg(nullptr) == ENC_E_INVALID_ARG);
  {
    encoder_cfg b = full;
    b.n_heads = 19;
    EXPECT(encoder_validate_cfg(&b) == ENC_E_INVALID_ARG);
    b = full;
    b.conv_channels = 16384;
    b.dtype = ENC_F32;
    EXPECT(encoder_validate_cfg(&b) == ENC_E_INVALID_ARG);
    b = full;
    b.sample_rate = 44100;
    EXPECT(encoder_validate_cfg(&b) == ENC_E_UNSUPPORTED);
    b = full;
    b.max_tokens_per_pass = -1;
    EXPECT(encoder_validate_cfg(&b) == ENC_E_INVALID_ARG);
  }
  int64_t nf = 0;
  EXPECT(encoder_weight_count(&full, &nf) == ENC_OK && nf == 698258816);
  EXPECT(encoder_weight_count(&tiny, &nf) == ENC_OK && nf == 3500160);
  EXPECT(encoder_weight_count(&full, nullptr) == ENC_E_INVALID_ARG);
  for (int64_t n : {201LL, 16000LL, 480000LL, 1024000LL, 57600000LL, 127999LL, 128001LL}) {
    int64_t f = 0;
    EXPECT(encoder_output_frames(&full, n, &f) == ENC_OK && f >= 1);
  }
  {
    int64_t f = 0;
    EXPECT(encoder_output_frames(&full, 200, &f) == ENC_E_INVALID_ARG);
    EXPECT(encoder_output_frames(&full, 480000, nullptr) == ENC_E_INVALID_ARG);
    int32_t nw = 0;
    EXPECT(encoder_plan_windows(&full, 480000, 0, nullptr, 0, &nw) == ENC_E_INVALID_ARG);
    EXPECT(encoder_plan_windows(&full, 480000, 2, nullptr, 3, &nw) == ENC_E_INVALID_ARG);
  }

  std::mt19937_64 rng(7);
  plans(full, {480000}, 0);
  plans(full, {57600000}, 1);
  plans(full, {57600000}, 8);
  plans(full, {2405920}, 2);
  plans(full, std::vector<int64_t>(16, 480000), 0);
  plans(full, std::vector<int64_t>(200, 80000), 0);
  plans(full, std::vector<int64_t>(113, 16000), 0);
  plans(full, {480000, 200}, 0);   // a clip too short: rejected
  plans(full, {480000, 480000}, 1);  // long mode takes one recording: rejected
  plans(tiny, {201, 201, 64000}, 0);
  for (int r = 0; r < 20; ++r) {
    std::vector<int64_t> lens(1 + rng() % 300);
    for (auto& v : lens) v = 201 + (int64_t)(rng() % 640000);
    encoder_cfg c = (r & 1) ? full : tiny;
    c.max_tokens_per_pass = (int64_t[]){0, 500, 3000, 8192, 100000}[r % 5];
    plans(c, lens, 0);
  }
  {
    int32_t np = 0;
    const int64_t one = 480000;
    EXPECT(encoder_plan_passes(&full, nullptr, 1, 0, nullptr, 0, &np) == ENC_E_INVALID_ARG);
    EXPECT(encoder_plan_passes(&full, &one, 1, -1, nullptr, 0, &np) == ENC_E_INVALID_ARG);
    EXPECT(encoder_plan_passes(&full, &one, 1, 0, nullptr, 2, &np) == ENC_E_INVALID_ARG);
    EXPECT(encoder_plan_passes(&full, &one, 1, 0, nullptr, 0, nullptr) == ENC_E_INVALID_ARG);
    EXPECT(encoder_plan_passes(&full, &one, 1, 11, nullptr, 0, &np) == ENC_E_INVALID_ARG);
  }

  // int4 quantiser: exact-size outputs
  for (auto nk : {std::pair<int64_t, int64_t>{3, 128}, {37, 1280}, {64, 2048}}) {
    const int64_t N = nk.first, K = nk.second;
    float* w = new float[(size_t)(N * K)];
    std::normal_distribution<float> nd(0.0f, 0.02f);
    for (int64_t i = 0; i < N * K; ++i) w[i] = nd(rng);
    for (int64_t i = 0; i < 128; ++i) w[i] = 0.0f;  // an all-zero group
    uint8_t* q = new uint8_t[(size_t)(N * K / 2)];
    uint16_t* s = new uint16_t[(size_t)(N * K / 128)];
    EXPECT(encoder_quantize_int4(w, N, K, q, s) == ENC_OK);
    EXPECT(s[0] == 0 && q[0] == 0);
    delete[] w;
    delete[] q;
    delete[] s;
  }
  {
    float w[4] = {0, 0, 0, 0};
    uint8_t q[2];
    uint16_t s[1];
    EXPECT(encoder_quantize_int4(w, 1, 100, q, s) == ENC_E_INVALID_ARG);
    EXPECT(encoder_quantize_int4(nullptr, 1, 128, q, s) == ENC_E_INVALID_ARG);
  }
  // conditioning lengths
  for (int32_t fs : {8000, 11025, 16000, 22050, 44100, 48000, 96000, 192000}) {
    int64_t n = 0;
    EXPECT(encoder_conditioned_length(1234567, fs, &n) == ENC_OK && n > 0);
  }
  {
    int64_t n = 0;
    EXPECT(encoder_conditioned_length(1000, 44101, &n) == ENC_E_UNSUPPORTED);
    EXPECT(encoder_conditioned_length(0, 16000, &n) == ENC_E_INVALID_ARG);
    EXPECT(encoder_conditioned_length(10, 16000, nullptr) == ENC_E_INVALID_ARG);
  }
  // create rejects a blob of the wrong size before touching a device
  {
    float* blob = new float[1000];
    std::memset(blob, 0, 1000 * sizeof(float));
    encoder* e = nullptr;
    EXPECT(encoder_create(blob, 1000, &tiny, &e) == ENC_E_INVALID_ARG && e == nullptr);
    EXPECT(std::strstr(encoder_last_error(), "config needs") != nullptr);
    EXPECT(encoder_create(nullptr, 3500160, &tiny, &e) == ENC_E_INVALID_ARG);
    delete[] blob;
  }
  // handle-less calls are rejected without a device
  EXPECT(encoder_forward(nullptr, nullptr, 1000, 1, nullptr, nullptr) == ENC_E_INVALID_ARG);
  EXPECT(encoder_memory_stats(nullptr, nullptr, nullptr) == ENC_E_INVALID_ARG);
  encoder_destroy(nullptr);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("host entry points: all checks passed\n");
  return 0;
}
