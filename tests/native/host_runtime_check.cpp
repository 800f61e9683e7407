// Drives the host side of libpld (sizing, validation, argument checks) without a GPU, for a
// build with AddressSanitizer and UndefinedBehaviorSanitizer on the host code. Prints the
// workspace size of each named workload and the outcome of a seeded fuzz of configuration
// fields; any sanitizer report aborts the program.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pld.h"

static pld_config base(int kind) {
  pld_config c;
  memset(&c, 0, sizeof(c));
  c.eps = 1e-6;
  c.rope_base = 10000.0;
  c.ffn_kind = PLD_FFN_MOE;
  switch (kind) {
    case 1:   // tiny dense MHA
      c.attn_kind = PLD_ATTN_GQA; c.wfmt = PLD_WFMT_BF16; c.hidden = 256; c.n_heads = 4; c.n_kv_heads = 4;
      c.head_dim = 64; c.ffn_kind = PLD_FFN_DENSE; c.inter = 1024; c.max_seq = 256;
      break;
    case 2:   // GQA MoE bf16
      c.attn_kind = PLD_ATTN_GQA; c.wfmt = PLD_WFMT_BF16; c.hidden = 4096; c.n_heads = 32; c.n_kv_heads = 8;
      c.head_dim = 128; c.inter = 1536; c.n_experts = 64; c.top_k = 8; c.n_shared = 1; c.max_seq = 8256;
      break;
    case 3: case 5: case 7:   // MLA FP8 (5: with the LM head, 7: LUT3 experts)
      c.attn_kind = PLD_ATTN_MLA; c.wfmt = PLD_WFMT_FP8_BLOCK128; c.hidden = 6144; c.n_heads = 64; c.q_lora = 1536;
      c.kv_lora = 512; c.rope_dim = 64; c.nope_dim = 128; c.v_dim = 128; c.inter = 2048; c.n_experts = 256;
      c.top_k = 8; c.n_shared = 1; c.router_kind = PLD_ROUTER_SIGMOID_BIAS; c.max_seq = 8256;
      if (kind == 5) { c.max_seq = 8456; c.vocab = 32768; }
      if (kind == 7) c.expert_wfmt = PLD_WFMT_LUT3;
      break;
    case 4:   // sparse MLA bf16
      c.attn_kind = PLD_ATTN_MLA; c.wfmt = PLD_WFMT_BF16; c.hidden = 4096; c.n_heads = 32; c.q_lora = 1536;
      c.kv_lora = 512; c.rope_dim = 64; c.nope_dim = 128; c.v_dim = 128; c.index_heads = 8; c.index_dim = 64;
      c.index_topk = 2048; c.inter = 1536; c.n_experts = 64; c.top_k = 8; c.n_shared = 1; c.max_seq = 32832;
      break;
    case 6:   // KDA
      c.attn_kind = PLD_ATTN_KDA; c.wfmt = PLD_WFMT_FP8_BLOCK128; c.hidden = 6144; c.n_heads = 32; c.head_dim = 128;
      c.kda_rank = 128; c.conv_width = 4; c.inter = 2048; c.n_experts = 256; c.top_k = 8; c.n_shared = 1;
      c.router_kind = PLD_ROUTER_SIGMOID_BIAS; c.max_seq = 8256;
      break;
  }
  return c;
}

int main() {
  for (int kind = 1; kind <= 7; kind++) {
    pld_config c = base(kind);
    printf("c%d %zu %zu\n", kind, pld_workspace_bytes_for_cus(&c, 1, 256), pld_workspace_bytes_for_cus(&c, 24, 256));
  }
  // seeded fuzz: one or two fields of a valid configuration set to arbitrary values
  uint64_t s = 12345;
  auto next = [&]() { s = s * 6364136223846793005ull + 1442695040888963407ull; return (uint32_t)(s >> 32); };
  int accepted = 0, total = 0;
  for (int i = 0; i < 20000; i++) {
    pld_config c = base(1 + next() % 7);
    int32_t* f = reinterpret_cast<int32_t*>(&c);
    const int nf = (int)(offsetof(pld_config, eps) / sizeof(int32_t));
    for (int k = 0; k < 1 + (int)(next() % 2); k++) {
      const uint32_t r = next();
      f[next() % nf] = (r & 3) == 0 ? (int32_t)r : (r & 3) == 1 ? -(int32_t)(r % 1000) : (int32_t)(r % 70000);
    }
    if (next() % 8 == 0) c.eps = (next() & 1) ? -1.0 : 1e300;
    const int cus = (next() & 1) ? 256 : (int)(next() % 1024) - 8;
    const size_t b = pld_workspace_bytes_for_cus(&c, (int32_t)(next() % 64) - 4, cus);
    accepted += b > 0;
    total++;
  }
  printf("fuzz %d of %d accepted\n", accepted, total);
  // argument checks that return before any device work
  pld_handle* h = nullptr;
  pld_config c = base(2);
  int ok = decode_layer_init(&c, 1, nullptr, nullptr, nullptr, nullptr, 0, &h) == PLD_E_INVALID && !h;
  ok = ok && decode_layer_init(nullptr, 1, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == PLD_E_INVALID;
  ok = ok && decode_step(nullptr, 0, nullptr, 0, nullptr, nullptr) == PLD_E_INVALID;
  ok = ok && decode_layers_persistent(nullptr, nullptr, nullptr) == PLD_E_INVALID;
  ok = ok && decode_speculative(nullptr, nullptr, nullptr, nullptr) == PLD_E_INVALID;
  ok = ok && decode_poll_status(nullptr, nullptr) == PLD_E_INVALID && decode_reset(nullptr) == PLD_E_INVALID;
  ok = ok && pld_set_test_hooks(nullptr, 0, 0) == PLD_E_INVALID && pld_set_watchdog_us(nullptr, 1) == PLD_E_INVALID;
  ok = ok && pld_debug_buffer(nullptr, "a", nullptr, nullptr) == PLD_E_INVALID;
  for (int code = -8; code <= 1; code++) ok = ok && pld_status_string((pld_status)code) != nullptr;
  decode_layer_destroy(nullptr);
  printf("args_ok %d\n", ok);
  return 0;
}
