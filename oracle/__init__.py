"""CPU oracle for the MoE routing / load-balance / dispatch path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import anything from this package.  The
GPU library (``load_balanced_expert_amd``) never imports it, and this package
never imports the GPU library: the two share no code.  The only shared module
is ``workloads`` (seeded random inputs, no arithmetic of the method).

Everything here is plain numpy / scipy, in float64 unless the pages fix the
precision (the Loss-Free bias state and the Quantile-Balancing duals are fp32
state and are computed in fp32; see the docstrings).  Each function cites the
page passage it follows, by page title and section:

* [Switch review]  "Switch Transformers 논문 리뷰: 1.6조 파라미터 MoE 모델의 Sparse
  Routing 기법 완전 분석" (tildalice.io)
* [Switch impl]    "Switch Transformer를 구현 관점에서 읽기: Top-1 라우팅과 Expert 병렬
  처리" (molayo1419.me)
* [MoE tour 6]     "MoE环游记：6、最优分配促均衡" (kexue.fm/archives/11619), read in
  its Korean translation "MoE 환유기: 6, 최적 할당으로 균형 촉진"
* [Qwen global]    "Qwen 글로벌-배치 로드 밸런스 MoE LLM 훈련" (agentlenshq.com)

Parity status of each part is recorded in the module docstrings.  Every
function is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_*.py``.
"""
from . import router, stats, dispatch, expert, balance  # noqa: F401
from . import backward  # noqa: F401,E402
