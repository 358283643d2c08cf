"""Plain fp64 CPU oracle for hybrid compressed attention (CSA + HCA).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package. The HIP product path
never calls it, and this package imports nothing from the HIP path.

Sources (cited by title and section throughout):
  [P5] "DeepSeek-V4가 이차적 어텐션 비용 없이 백만 토큰 컨텍스트를 달성하는 방법"
       (molayo1419.me), section "두 가지 압축 전략: CSA 및 HCA": CSA pools 4
       consecutive tokens by softmax weights, an FP4 lightning indexer scores the
       pooled entries and keeps the top ~128, a sliding window runs alongside;
       HCA pools 128 tokens and attends densely; both use shared-KV MQA with
       partial RoPE.
  [P3] "딥시크 V4 분석: CSA·HCA 어텐션으로 100만 토큰 컨텍스트를 저비용에 구현한
       방법" (allinfo.ai.kr), sections "쉽게 이해하기" (learned 4->1 entries,
       128->1 dense branch, 128-token window) and "주요 인사이트" (1:1 interleave).
  [P1] "Is DeepSeek v4 (Flash) really extremely cheap to run? If yes, how?"
       (aiwitness.kr digest), section "주요 댓글": the indexer of DSA runs over
       all stored KV and full attention runs only on what it picks.
  [P4] jjy0501.blogspot.com post on DeepSeek V4.1 Flash: the local SWA cache
       holds the latest 128 tokens.

Readings of the pages (where they are silent) are stated in each module.

Modules:
  formats    storage decoders/encoders (bf16, OCP e4m3fn, OCP MXFP4)
  rope       partial rotary embedding, adjacent-pair form
  compress   softmax pooling of m-token blocks (CSA m=4, HCA m=128)
  indexer    lightning-indexer scores (exact)
  topk       top-k by (score desc, index asc)
  attention  joint-softmax MQA attention over entries + window
  hybrid     decode loop with ring buffer and periodic re-compression
"""
from . import formats, rope, compress, indexer, topk, attention, hybrid  # noqa: F401
