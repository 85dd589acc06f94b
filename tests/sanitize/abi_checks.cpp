// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer around the library's host code (the planner,
// workspace sizing and argument validation); no device is needed, since every
// call here either only sizes a workspace or is rejected before anything is
// enqueued.  Device pointers are fake non-NULL addresses that are never read.
// Exit status 0 when every call returned what is expected.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "vb.h"

namespace {

int failures = 0;

void expect(const char* what, vb_status got, vb_status want, const char* msg = nullptr) {
  const bool ok = got == want && (!msg || std::strstr(vb_last_error(), msg));
  if (!ok) {
    std::printf("FAIL %s: status %d (want %d), message '%s'\n", what, (int)got, (int)want, vb_last_error());
    ++failures;
  } else {
    std::printf("ok   %s\n", what);
  }
}

const float* fake(uintptr_t a) { return reinterpret_cast<const float*>(a); }

vb_node node(int op, int in0, int c, int h = 1, int w = 1, const float* W = nullptr, const float* b = nullptr) {
  vb_node n{};
  n.op = op;
  n.in0 = in0;
  n.in1 = -1;
  n.c = c;
  n.h = h;
  n.w = w;
  n.weight = W;
  n.bias = b;
  return n;
}

vb_node conv(int in0, int c, int h, int w, int k, int s, int p) {
  vb_node n = node(VB_CONV2D, in0, c, h, w, fake(256), fake(512));
  n.kh = n.kw = k;
  n.stride = s;
  n.pad = p;
  return n;
}

vb_node add(int a, int b, int c, int h, int w) {
  vb_node n = node(VB_ADD, a, c, h, w);
  n.in1 = b;
  return n;
}

// A residual network like the measured one at a smaller width: stem, stages of
// basic blocks (stride-2 conv_a and 1x1 projection at a stage change), GAP, FC.
std::vector<vb_node> resnet(int c0, int stages, int blocks) {
  std::vector<vb_node> g;
  g.push_back(node(VB_INPUT, -1, 3, 32, 32));
  g.push_back(conv(0, c0, 32, 32, 3, 1, 1));
  g.push_back(node(VB_RELU, 1, c0, 32, 32));
  int cur = 2, c = c0, h = 32;
  for (int s = 0; s < stages; ++s) {
    for (int b = 0; b < blocks; ++b) {
      const bool down = s > 0 && b == 0;
      const int co = down ? 2 * c : c, ho = down ? h / 2 : h;
      g.push_back(conv(cur, co, ho, ho, 3, down ? 2 : 1, 1));
      g.push_back(node(VB_RELU, (int)g.size() - 1, co, ho, ho));
      g.push_back(conv((int)g.size() - 1, co, ho, ho, 3, 1, 1));
      const int main = (int)g.size() - 1;
      int skip = cur;
      if (down) {
        g.push_back(conv(cur, co, ho, ho, 1, 2, 0));
        skip = (int)g.size() - 1;
      }
      g.push_back(add(main, skip, co, ho, ho));
      g.push_back(node(VB_RELU, (int)g.size() - 1, co, ho, ho));
      cur = (int)g.size() - 1;
      c = co;
      h = ho;
    }
  }
  g.push_back(node(VB_GAP, cur, c));
  g.push_back(node(VB_LINEAR, (int)g.size() - 1, 10, 1, 1, fake(256), fake(512)));
  return g;
}

}  // namespace

int main() {
  size_t n = 0;
  // -- workspace sizing over every method on an MLP, a CNN and a residual net
  std::vector<vb_node> mlp = {node(VB_INPUT, -1, 4), node(VB_LINEAR, 0, 5, 1, 1, fake(16), fake(32)),
                              node(VB_RELU, 1, 5), node(VB_LINEAR, 2, 3, 1, 1, fake(16), fake(32))};
  vb_graph gm{(int32_t)mlp.size(), mlp.data()};
  const int methods[] = {VB_METHOD_IBP, VB_METHOD_CROWN, VB_METHOD_HYBRID, VB_METHOD_CROWN | VB_INTERSECT_IBP,
                         VB_METHOD_HYBRID | VB_INTERSECT_IBP, VB_METHOD_CROWN | VB_UNSTABLE_ONLY,
                         VB_METHOD_CROWN | VB_ALPHA_ROWS};
  for (int method : methods) {
    char what[64];
    std::snprintf(what, sizeof what, "mlp workspace, method %d", method);
    expect(what, vb_workspace_size(&gm, 3, 2, method, (method & 3) == VB_METHOD_HYBRID ? 2 : 0, &n), VB_OK);
  }
  std::vector<vb_node> cnn = {node(VB_INPUT, -1, 3, 32, 32), conv(0, 16, 32, 32, 3, 1, 1), node(VB_RELU, 1, 16, 32, 32),
                              conv(2, 16, 16, 16, 3, 2, 1),   node(VB_RELU, 3, 16, 16, 16),  node(VB_FLATTEN, 4, 4096),
                              node(VB_LINEAR, 5, 10, 1, 1, fake(256), fake(512))};
  vb_graph gc{(int32_t)cnn.size(), cnn.data()};
  for (int method : methods) {
    char what[64];
    std::snprintf(what, sizeof what, "cnn workspace, method %d", method);
    expect(what, vb_workspace_size(&gc, 2, 9, method, (method & 3) == VB_METHOD_HYBRID ? 2 : 0, &n), VB_OK);
  }
  std::vector<vb_node> res = resnet(32, 3, 2);
  vb_graph gr{(int32_t)res.size(), res.data()};
  int region = 0;
  for (int k = (int)res.size() - 1; k > 0; --k)  // input of the last stage: the ReLU before its first conv
    if (res[k].op == VB_CONV2D && res[k].stride == 2) {
      region = res[k].in0;
      break;
    }
  for (int method : methods) {
    char what[64];
    std::snprintf(what, sizeof what, "residual workspace, method %d", method);
    expect(what, vb_workspace_size(&gr, 4, 99, method, (method & 3) == VB_METHOD_HYBRID ? region : 0, &n), VB_OK);
  }
  size_t nb = 0;
  expect("branch-and-bound workspace", vb_bab_workspace_size(&gm, 2, 8, &nb), VB_OK);
  // -- graph errors
  std::vector<vb_node> bad = mlp;
  bad[1].weight = nullptr;
  vb_graph gb{(int32_t)bad.size(), bad.data()};
  expect("NULL weight", vb_workspace_size(&gb, 2, 2, 1, 0, &n), VB_EINVAL, "weight is NULL");
  bad = mlp;
  bad[1].in0 = 3;
  expect("bad input index", vb_workspace_size(&gb, 2, 2, 1, 0, &n), VB_ESHAPE);
  bad = mlp;
  bad[2].c = 4;
  expect("relu shape", vb_workspace_size(&gb, 2, 2, 1, 0, &n), VB_ESHAPE, "relu shape");
  expect("bad method", vb_workspace_size(&gm, 2, 2, 7, 0, &n), VB_EINVAL);
  expect("zero batch", vb_workspace_size(&gm, 0, 2, 1, 0, &n), VB_EINVAL);
  std::vector<vb_node> cv = {node(VB_INPUT, -1, 3, 8, 8), conv(0, 4, 5, 4, 3, 2, 1)};
  vb_graph gv{(int32_t)cv.size(), cv.data()};
  expect("conv output shape", vb_workspace_size(&gv, 2, 0, 0, 0, &n), VB_ESHAPE, "conv output");
  // -- entry points reject bad arguments before enqueuing anything
  const float* nulls[4] = {nullptr, nullptr, nullptr, nullptr};
  float* const* nullw = const_cast<float* const*>(reinterpret_cast<const float* const*>(nulls));
  void* ws = const_cast<float*>(fake(64));
  expect("crown: NULL centre", vb_crown(&gm, 2, nullptr, nullptr, 0.1f, 1, 0, nullw, nullw, nullptr, 0, nullptr,
                                        nullptr, nullptr, nullptr, ws, 1 << 20, nullptr),
         VB_EINVAL);
  expect("crown: NULL bounds storage", vb_crown(&gm, 2, fake(64), nullptr, 0.1f, 1, 0, nullw, nullw, nullptr, 0,
                                                nullptr, nullptr, nullptr, nullptr, ws, 1 << 20, nullptr),
         VB_EINVAL, "bounds storage");
  const float* bd[4] = {nullptr, fake(64), fake(64), fake(64)};
  float* const* bdw = const_cast<float* const*>(reinterpret_cast<const float* const*>(bd));
  expect("crown: workspace too small", vb_crown(&gm, 2, fake(64), nullptr, 0.1f, 1, 0, bdw, bdw, fake(64), 2, nullptr,
                                                nullptr, const_cast<float*>(fake(64)), const_cast<float*>(fake(64)),
                                                ws, 16, nullptr),
         VB_ENOMEM, "too small");
  expect("ibp: negative eps", vb_ibp(&gm, 2, fake(64), nullptr, -1.f, nullw, nullw, nullptr, 0, nullptr, nullptr,
                                     nullptr, 0, nullptr),
         VB_EINVAL);
  expect("crown_backward: stop >= start", vb_crown_backward(&gm, 2, 1, 1, nullptr, 0, bd, bd, nullptr, nullptr,
                                                            fake(64), nullptr, 0.1f, nullptr, nullptr, nullptr,
                                                            nullptr, ws, 1 << 20, nullptr),
         VB_EINVAL);
  expect("crown_backward: workspace checked first",
         vb_crown_backward(&gm, 2, 3, 0, nullptr, 0, bd, bd, nullptr, nullptr, fake(64), nullptr, 0.1f,
                           const_cast<float*>(fake(64)), const_cast<float*>(fake(64)), nullptr, nullptr, ws, 64,
                           nullptr),
         VB_ENOMEM, "too small");
  expect("concretize: zero rows", vb_concretize(0, 4, 1, fake(64), nullptr, fake(64), nullptr, 0.1f, nullptr,
                                                nullptr, nullptr),
         VB_EINVAL);
  std::vector<vb_node> relu_in = {node(VB_INPUT, -1, 4), node(VB_LINEAR, 0, 4, 1, 1, fake(16), fake(32)),
                                  node(VB_RELU, 0, 4)};
  vb_graph gi{(int32_t)relu_in.size(), relu_in.data()};
  const float* b3[3] = {nullptr, fake(64), fake(64)};
  float* const* b3w = const_cast<float* const*>(reinterpret_cast<const float* const*>(b3));
  expect("ibp: ReLU on the input", vb_ibp(&gi, 2, fake(64), nullptr, 0.1f, b3w, b3w, nullptr, 0, nullptr, nullptr,
                                          nullptr, 0, nullptr),
         VB_EUNSUPPORTED);
  int32_t ver[2];
  expect("verify: bad m", vb_verify(2, 0, fake(64), ver, nullptr, nullptr), VB_EINVAL);
  std::printf("%d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
